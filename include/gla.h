/*
 * gla.h -- C ABI of the MI355X (gfx950) gated linear-attention forward library.
 *
 * The operation is the gated linear-attention token mixer that carries the
 * O(N) part of the hybrid video DiT described in "SANA-Video 2.0: Hybrid
 * Linear Attention with Attention Residuals for Efficient Video Generation"
 * (project page, section "Hybrid Linear-Softmax Attention"). For each batch b
 * and head h, over tokens t = 0..N-1 with head dimension d:
 *
 *   phi(x) = max(x, 0),  sigma(x) = 1 / (1 + exp(-x))
 *   state    S in R^{d x d} (S[i][j]: i = key feature, j = value feature)
 *   normaliser z in R^d
 *   o_t = sigma(g_t) (.) (phi(q_t)^T S) / (phi(q_t)^T z + eps)
 *
 * Two modes:
 *  - bidirectional: one state over the whole sequence,
 *      S = sum_t phi(k_t) v_t^T, z = sum_t phi(k_t);
 *  - frame-causal (block-causal over video frames of T tokens each, F frames):
 *      S_f = gamma_f S_{f-1} + sum_{t in frame f} phi(k_t) v_t^T,
 *      z_f = gamma_f z_{f-1} + sum_{t in frame f} phi(k_t),
 *      S_{-1} = S_in (or 0), and every token of frame f reads S_f, z_f.
 *    The fixed D x D state and its additive per-block update are the block KV
 *    cache of "SANA-Video: Efficient Video Generation with Block Linear
 *    Diffusion Transformer" (ICLR 2026 oral, block KV cache passage); the
 *    per-frame decay gamma_f follows the frame-wise decay gates of the
 *    "SANA-WM" analysis page (method components).
 *
 * Conventions for every entry point:
 *  - Layout: q, k, v, g, o are [B][H][N][d] row-major (each (b, h) slab is a
 *    contiguous N x d matrix; N = F * T in frame-causal mode). gamma is
 *    [B][H][F] float32; S_* are [B][H][d][d] float32; z_* are [B][H][d] float32.
 *  - dtype: GLA_F32 (float32 inputs and output) or GLA_BF16 (bfloat16 inputs
 *    and output, float32 accumulation; the output is rounded to nearest even).
 *  - Supported head dimensions: d in {16, 32, 64, 128}.
 *  - Pointers are device memory of the current HIP device, owned by the
 *    caller. The entry points never allocate, free or synchronise; all work is
 *    enqueued asynchronously on `stream` (a hipStream_t; NULL is the default
 *    stream). A call enqueues kernel launches only (no memset, copy or
 *    synchronisation), so it can be captured into a HIP graph and replayed.
 *    The library keeps no state between calls (apart from the optional
 *    timing session below): calls from several threads or on several
 *    streams may run at once when their outputs and workspaces are disjoint.
 *    Tensor pointers must be 16-byte aligned, gamma 4-byte aligned, the
 *    workspace 256-byte aligned.
 *  - Aliasing: S_out may equal S_in and z_out may equal z_in (in-place
 *    update). No other overlap is allowed (checked: GLA_ERR_ALIAS).
 *  - Errors: every argument is validated on the host before anything is
 *    enqueued; on any status other than GLA_OK nothing was launched. A failed
 *    launch returns GLA_ERR_HIP. Faults during execution surface at the
 *    caller's next synchronisation. gla_last_error() gives a thread-local
 *    message for the last non-OK status. No C++ exception crosses the ABI.
 *  - Determinism: results are bitwise identical from run to run for the same
 *    inputs and shapes (fixed reduction order, no floating-point atomics).
 *  - Empty inputs: B, H, N, F or T may be 0; the call then only produces the
 *    state outputs implied by the definition (e.g. F = 0 gives S_out = S_in).
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gla_status {
  GLA_OK = 0,
  GLA_ERR_NULL = 1,        /* a required pointer is NULL, or only one of a pair is given */
  GLA_ERR_SHAPE = 2,       /* negative or inconsistent sizes, or sizes that overflow */
  GLA_ERR_UNSUPPORTED = 3, /* head dimension or dtype not supported */
  GLA_ERR_ALIGN = 4,       /* pointer misaligned */
  GLA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the *_workspace query */
  GLA_ERR_VALUE = 6,       /* eps negative or not finite */
  GLA_ERR_HIP = 7,         /* the HIP runtime reported an error at launch */
  GLA_ERR_ALIAS = 8,       /* an output overlaps an input or the workspace */
  /* Not statuses: these two give the type the range of a 32-bit int, so that
   * any int a C caller passes (gla_status_string) is a value of the type in
   * the C++ implementation too, which then maps unknown values to a message. */
  GLA_STATUS_RANGE_MIN_ = -2147483647 - 1,
  GLA_STATUS_RANGE_MAX_ = 2147483647
} gla_status;

typedef enum gla_dtype {
  GLA_F32 = 0,
  GLA_BF16 = 1,
  /* Not dtypes: the range of a 32-bit int, so that an unknown value a C caller
   * passes is still a value of the type on the C++ side, where it is refused
   * with GLA_ERR_UNSUPPORTED. */
  GLA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  GLA_DTYPE_RANGE_MAX_ = 2147483647
} gla_dtype;

/* Workspace bytes needed by the matching call for these sizes (0 if none).
 * Returns 0 for invalid sizes as well; the call itself reports those. */
size_t gla_fwd_bidir_workspace(int B, int H, int64_t N, int d);
size_t gla_fwd_framecausal_workspace(int B, int H, int F, int T, int d);
size_t gla_state_carry_workspace(int B, int H, int F, int T, int d);

/* Bidirectional (whole-sequence, non-causal) gated linear attention.
 * Defining passages: the O(N) gated linear-attention mixer of the hybrid DiT
 * ("SANA-Video 2.0" project page, section "Hybrid Linear-Softmax Attention"),
 * in the form a denoising DiT applies it to a clip it diffuses as a whole:
 * every token reads the one state summed over all tokens ("SANA-Video" ICLR
 * 2026 oral talk: the video model's linear-attention DiT is the image model's,
 * and a block is diffused jointly, all of its tokens seeing one another).
 * Equals the frame-causal mode's last frame with gamma = 1 (no decay).
 * Reads q, k, v, g [B][H][N][d]; writes o [B][H][N][d]. The workspace holds
 * one fp32 state of d*d + d floats per (slab, part); nothing in it needs to
 * be initialised. */
gla_status gla_fwd_bidir(const void *q, const void *k, const void *v, const void *g, void *o,
                         int B, int H, int64_t N, int d, gla_dtype dt, float eps, void *ws,
                         size_t ws_bytes, void *stream);

/* Frame-causal gated linear attention with per-frame decay gamma [B][H][F].
 * Defining passages: block-causal linear attention over video frames with a
 * constant-size carried state ("SANA-Video" ICLR 2026 oral talk, block-causal
 * linear attention and block KV cache passages), gated by a per-frame decay
 * ("SANA-WM" analysis page, method components: frame-wise decay gates).
 * S_in/z_in: carried-in state (both NULL: zero state). S_out/z_out: state after
 * the last frame (both NULL: not written). o [B][H][F*T][d]. The workspace
 * holds fp32 states of d*d + d floats per (slab, frame, part) plus one per
 * (slab, group of frames); nothing in it needs to be initialised. */
gla_status gla_fwd_framecausal(const void *q, const void *k, const void *v, const void *g,
                               const float *gamma, const float *S_in, const float *z_in,
                               void *o, float *S_out, float *z_out, int B, int H, int F, int T,
                               int d, gla_dtype dt, float eps, void *ws, size_t ws_bytes,
                               void *stream);

/* Block-cache commit: the state after F more frames, from k, v and gamma only
 * (no queries, no output). Defining passage: the block KV cache of the
 * "SANA-Video" ICLR 2026 oral talk (block KV cache passage): the D x D state
 * of a finished block is cached and the next block's KV contribution is added
 * to it; with the frame-wise decay of the "SANA-WM" analysis page (method
 * components), S_out = S_{F-1} of the frame-causal recurrence above, started
 * from S_in. Equals the S_out/z_out of gla_fwd_framecausal on the same
 * inputs. S_out and z_out are required (S_out may be S_in). */
gla_status gla_state_carry(const void *k, const void *v, const float *gamma, const float *S_in,
                           const float *z_in, float *S_out, float *z_out, int B, int H, int F,
                           int T, int d, gla_dtype dt, void *ws, size_t ws_bytes, void *stream);

/* ---- the frame-causal forward without a workspace argument ------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * gla_fwd_framecausal_noalloc computes exactly gla_fwd_framecausal (the same
 * kernels and plan: the results are bitwise those of gla_fwd_framecausal), with
 * its workspace in a static device array of GLA_NOALLOC_SCRATCH_BYTES inside the
 * library instead of a caller's buffer. The call allocates and frees nothing.
 *  - Limit: sizes whose gla_fwd_framecausal_workspace exceeds
 *    GLA_NOALLOC_SCRATCH_BYTES (256 MiB: the 720p/60s shape with H = 32,
 *    d = 64 needs 138 MiB; a 31-frame block at B = 2, H = 40, d = 128, 237 MiB)
 *    are refused with GLA_ERR_WORKSPACE before any HIP call.
 *  - Memory: every GPU the library runs this call on holds its own copy of the
 *    array until the process ends. The first call on a device looks up the
 *    array's device address there (hipGetSymbolAddress) and keeps it; a
 *    failure of that lookup returns GLA_ERR_HIP.
 *  - Concurrency: every call on one GPU uses that GPU's one array. Calls that
 *    overlap in time on one GPU (other threads, other streams) race on it and
 *    give undefined results: serialise them, e.g. on one stream. Nothing in the
 *    array needs to start at zero, and a call leaves it holding that call's
 *    per-frame states.
 *  - Arguments, validation and errors otherwise as gla_fwd_framecausal. */
#define GLA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

gla_status gla_fwd_framecausal_noalloc(const void *q, const void *k, const void *v,
                                       const void *g, const float *gamma, const float *S_in,
                                       const float *z_in, void *o, float *S_out, float *z_out,
                                       int B, int H, int F, int T, int d, gla_dtype dt,
                                       float eps, void *stream);

/* ---- backward pass ---------------------------------------------------------
 *
 * Gradients of the forward operation above for a loss L, given
 * dO = dL/do [B][H][N][d] (the input dtype) and, frame-causal only, the
 * optional dS_out = dL/dS_out and dz_out = dL/dz_out (fp32, both or neither;
 * NULL: zero). The pages state the forward only; these are its chain rule
 * (the derivative of ReLU taken as 0 at 0):
 *   dq, dk, dv, dg  [B][H][N][d], the input dtype, rounded from fp32 (on the
 *                   bf16 matrix-core path dg takes 1 - sigmoid(g) rounded to
 *                   fp16, about 11 significant bits, before the product);
 *   dgamma          [B][H][F] fp32 (frame-causal; NULL: not computed);
 *   dS_in, dz_in    fp32, dL/dS_in and dL/dz_in (frame-causal; both or neither;
 *                   with S_in NULL they are the gradients of a zero state).
 * For a stream run block by block, the backward of the last block is called
 * first with the final dS_out; its dS_in is the previous block's dS_out.
 *
 * The forward states are recomputed inside the call (q, k, v, g, gamma,
 * S_in, z_in are the forward's inputs). The workspace (the *_workspace
 * queries) holds one fp32 state per (slab, frame, part) twice over. Outputs
 * may overlap no input, other output or the workspace (GLA_ERR_ALIAS).
 * Conventions otherwise as above. */
size_t gla_bwd_framecausal_workspace(int B, int H, int F, int T, int d);
size_t gla_bwd_bidir_workspace(int B, int H, int64_t N, int d);

gla_status gla_bwd_framecausal(const void *q, const void *k, const void *v, const void *g,
                               const float *gamma, const float *S_in, const float *z_in,
                               const void *dO, const float *dS_out, const float *dz_out,
                               void *dq, void *dk, void *dv, void *dg, float *dgamma,
                               float *dS_in, float *dz_in, int B, int H, int F, int T, int d,
                               gla_dtype dt, float eps, void *ws, size_t ws_bytes, void *stream);

gla_status gla_bwd_bidir(const void *q, const void *k, const void *v, const void *g,
                         const void *dO, void *dq, void *dk, void *dv, void *dg, int B, int H,
                         int64_t N, int d, gla_dtype dt, float eps, void *ws, size_t ws_bytes,
                         void *stream);

/* ---- per-frame state record (training) -------------------------------------
 *
 * The frame-causal forward can record the state every frame reads, so that
 * its backward need not recompute the states from k, v and gamma (it skips
 * the kv and carry launches: about a sixth of the backward at 720p/60s).
 *
 * states [B][H][F][d*d + d] float32: for frame f, S_f (d x d row-major, rows
 * the key features) followed by z_f -- the state of the frame-causal
 * definition above, as the tokens of frame f read it.
 *
 * gla_fwd_framecausal_states: gla_fwd_framecausal that also writes states
 * (required when B*H*F > 0). The scan runs one frame at a time (the plain
 * call folds frames in groups), so o may differ from gla_fwd_framecausal's in
 * the last bits. Its workspace need is at most gla_fwd_framecausal_workspace.
 *
 * gla_bwd_framecausal_states: gla_bwd_framecausal given the states written by
 * gla_fwd_framecausal_states for the same q, k, v, g, gamma, S_in, z_in (S_in,
 * z_in are still read for dgamma of the first frame). The results are bitwise
 * those of gla_bwd_framecausal. The workspace holds the adjoint sums only
 * (gla_bwd_framecausal_states_workspace). states is an input: outputs may
 * not overlap it. Conventions otherwise as above. */
gla_status gla_fwd_framecausal_states(const void *q, const void *k, const void *v,
                                      const void *g, const float *gamma, const float *S_in,
                                      const float *z_in, void *o, float *S_out, float *z_out,
                                      float *states, int B, int H, int F, int T, int d,
                                      gla_dtype dt, float eps, void *ws, size_t ws_bytes,
                                      void *stream);

size_t gla_bwd_framecausal_states_workspace(int B, int H, int F, int T, int d);

gla_status gla_bwd_framecausal_states(const void *q, const void *k, const void *v,
                                      const void *g, const float *gamma, const float *S_in,
                                      const float *z_in, const float *states, const void *dO,
                                      const float *dS_out, const float *dz_out, void *dq,
                                      void *dk, void *dv, void *dg, float *dgamma, float *dS_in,
                                      float *dz_in, int B, int H, int F, int T, int d,
                                      gla_dtype dt, float eps, void *ws, size_t ws_bytes,
                                      void *stream);

/* ---- frame-wise Gated DeltaNet ----------------------------------------------
 *
 * The other linear mixer of the pages: the SANA-WM analysis page (method
 * components; claim checks) describes a frame-wise Gated DeltaNet -- decay
 * gates plus a delta-rule correction of the recurrent state, with keys scaled
 * by 1/sqrt(D S) -- and gives no equations. This library reads it as one block
 * delta-rule update per frame, every token of the frame measuring its
 * prediction error against the same decayed prior (S = tokens per frame):
 *   P_f = gamma_f S_{f-1}                 (S_{-1} = S_in, or 0)
 *   e_t = v_t - P_f^T (c k_t)             c = key_scale (1/sqrt(d T) reads the pages)
 *   S_f = P_f + sum_{t in f} beta_t (c k_t) e_t^T
 *   o_t = S_f^T q_t                       every token of frame f
 * There is no feature map, normaliser or gate: q, k, v are used as given.
 * q, k, v, o [B][H][F*T][d] (GLA_F32 or GLA_BF16, rounded to nearest even);
 * beta [B][H][F*T] fp32 write strengths (typically in [0, 1]); gamma [B][H][F]
 * fp32; S_in, S_out [B][H][d][d] fp32 (either may be NULL; S_out may be S_in).
 * q and o both NULL: the state only (a block-cache commit). key_scale must be
 * finite and > 0. Conventions otherwise as above; the workspace holds 2 d^2
 * floats per (slab, frame, part). */
size_t gla_gdn_framecausal_workspace(int B, int H, int F, int T, int d);

gla_status gla_gdn_framecausal(const void *q, const void *k, const void *v, const float *beta,
                               const float *gamma, const float *S_in, void *o, float *S_out,
                               int B, int H, int F, int T, int d, gla_dtype dt, float key_scale,
                               void *ws, size_t ws_bytes, void *stream);

/* ---- gated softmax anchor ------------------------------------------------------
 *
 * The layer the linear mixers alternate with. The SANA-Video 2.0 project page
 * ("Hybrid Linear-Softmax Attention") places a gated-softmax anchor in one
 * layer of every four, to restore full-rank token interactions; the SANA-WM
 * analysis page (deployment) gives the softmax layers attention-sink tokens
 * and a local temporal window, so that their memory and per-chunk latency stay
 * constant along a rollout. Neither page prints a formula. This library
 * computes, with whole frames visible and the gate of the linear layers,
 *   o_t = sigmoid(g_t) (.) sum_{s in V(t)} softmax_s(scale q_t . k_s) v_s
 * k, v: [B][H][F*T][d], F frames of T tokens. q, g, o: [B][H][Fq*T][d], the
 * tokens of the last Fq <= F key frames: query frame j is key frame
 * f = F - Fq + j (a streaming call passes [kept frames | new frames] as keys
 * and the new frames as queries). causal = 0: V(t) is every key. causal = 1:
 * V(t) is the key frames i <= f with i < n_sink (the sink frames) or
 * i > f - window (the local window, which ends with the query's own frame;
 * window <= 0: no limit). scale must be finite and > 0 (1/sqrt(d) is the
 * usual choice); n_sink >= 0. GLA_F32 or GLA_BF16 (o rounded to nearest even),
 * softmax and sums in fp32. No workspace. o may overlap no input
 * (GLA_ERR_ALIAS). Conventions otherwise as above.
 * Precision of the bf16 matrix-core path (d = 32, 64, 128): scores on bf16
 * matrix cores with fp32 sums; P V on fp16 matrix cores, V converted from bf16
 * (exact in fp16's range) and the probabilities rounded to fp16. A tile of
 * 128 queries whose visible keys have a largest |v| outside [2^-6, 65504] is
 * recomputed by a second launch with P V in bf16 and each probability split
 * into a bf16 hi + lo pair; that launch costs the other tiles one load each.
 * The first launch marks such a tile by writing a NaN with payload 1 (bf16
 * 0x7FC1) at its first output element, so o holds that value between the two
 * launches. */
gla_status gla_softmax_anchor(const void *q, const void *k, const void *v, const void *g, void *o,
                              int B, int H, int Fq, int F, int T, int d, gla_dtype dt, int causal,
                              int n_sink, int window, float scale, void *stream);

/* ---- strided tensors and fused 3D rotary positions ------------------------
 *
 * The *_ex entry points compute the same operation as the plain ones, with
 * two additions:
 *
 * 1. Any layout whose feature axis is contiguous. A gla_tensor describes a
 *    [B][H][N][d] tensor whose element (b, h, n, c) sits at
 *      data + b * stride_b + h * stride_h + n * stride_n + c
 *    (strides in elements, >= 0). Examples: [B][N][H][d] is stride_b = N*H*d,
 *    stride_h = d, stride_n = H*d; the q, k, v of a fused [B][N][3][H][d]
 *    projection are three such views with stride_n = 3*H*d, 1 apart in the
 *    "3" axis. Every row must start 16-byte aligned: data 16-byte aligned and
 *    each stride a multiple of 16 bytes. Inputs may share memory and may
 *    broadcast (a zero stride). The output may overlap no input, state or the
 *    workspace (checked on the address span of each view: GLA_ERR_ALIAS), and
 *    distinct (b, h, n) of it must be distinct rows (GLA_ERR_ALIAS). A NULL
 *    gla_tensor pointer, or a NULL data, is an absent tensor.
 *
 * 2. Optional 3D rotary positions (rope != NULL). The SANA-Video ICLR 2026
 *    oral talk (passage on temporal modeling) adds 3D RoPE to the linear
 *    attention without saying where it acts; this library takes the rotary
 *    linear attention of RoFormer (section 3.3): the numerator uses turned
 *    features, the normaliser does not,
 *      o_n = sigma(g_n) (.) (sum_s (R_n phi(q_n))^T (R_s phi(k_s)) v_s^T) /
 *            (phi(q_n)^T sum_s phi(k_s) + eps),
 *    with the sums running over the keys that token n sees (all keys, or the
 *    decayed frame-causal prefix) and R_n the rotation of token n's position.
 *    Token l of frame f sits at (t, y, x) = (frame_offset + f, l / grid_w,
 *    l % grid_w); T must equal grid_h * grid_w. Feature pairs (2p, 2p+1) form
 *    three consecutive sections of dim_t / 2, dim_h / 2 and dim_w / 2 pairs
 *    (dim_* even, >= 0, summing to d) that turn with t, y and x respectively;
 *    pair j of an m-pair section turns by the angle pos * theta^(-j / m):
 *    (a, b) -> (a cos - b sin, a sin + b cos). theta must be finite and > 0;
 *    |frame_offset| and F must be below 2^30. The carried state S of the
 *    frame-causal mode then holds turned keys at their absolute positions, so
 *    a stream continued block by block passes each block's first frame as its
 *    frame_offset. With the matrix-core kernels (bf16, d in {32, 64, 128})
 *    the per-workgroup table of turns must fit:
 *    1 + grid_h * dim_h / 2 + grid_w * dim_w / 2 + 8 * dim_t / 2 <= 3072,
 *    else GLA_ERR_UNSUPPORTED; there the turned features are rounded to bf16
 *    for the matrix cores.
 */
typedef struct gla_tensor {
  void *data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_n;
} gla_tensor;

typedef struct gla_rope3d {
  int32_t grid_h;       /* token rows per frame */
  int32_t grid_w;       /* tokens per row */
  int32_t frame_offset; /* temporal position of the call's frame 0 */
  int32_t dim_t;        /* features turning with the frame */
  int32_t dim_h;        /* features turning with the row */
  int32_t dim_w;        /* features turning with the column */
  double theta;         /* frequency base */
} gla_rope3d;

/* Workspace of gla_fwd_bidir_ex: with rope, that of gla_fwd_framecausal for
 * (B, H, F, T, d) (the positions need the frame structure); without, that of
 * gla_fwd_bidir for N = F * T. The other two *_ex calls take the workspace
 * of their plain counterparts. */
size_t gla_fwd_bidir_ex_workspace(int B, int H, int F, int T, int d, const gla_rope3d *rope);

/* gla_fwd_bidir over N = F * T tokens (F frames of T tokens: the frames only
 * place the rotary positions). */
gla_status gla_fwd_bidir_ex(const gla_tensor *q, const gla_tensor *k, const gla_tensor *v,
                            const gla_tensor *g, const gla_tensor *o, int B, int H, int F, int T,
                            int d, gla_dtype dt, float eps, const gla_rope3d *rope, void *ws,
                            size_t ws_bytes, void *stream);

/* gla_fwd_framecausal with strided tensors and optional rotary positions. */
gla_status gla_fwd_framecausal_ex(const gla_tensor *q, const gla_tensor *k, const gla_tensor *v,
                                  const gla_tensor *g, const float *gamma, const float *S_in,
                                  const float *z_in, const gla_tensor *o, float *S_out,
                                  float *z_out, int B, int H, int F, int T, int d, gla_dtype dt,
                                  float eps, const gla_rope3d *rope, void *ws, size_t ws_bytes,
                                  void *stream);

/* gla_state_carry with strided tensors and optional rotary positions (the
 * state then holds turned keys: it matches gla_fwd_framecausal_ex's S_out). */
gla_status gla_state_carry_ex(const gla_tensor *k, const gla_tensor *v, const float *gamma,
                              const float *S_in, const float *z_in, float *S_out, float *z_out,
                              int B, int H, int F, int T, int d, gla_dtype dt,
                              const gla_rope3d *rope, void *ws, size_t ws_bytes, void *stream);

/* Training on strided tensors, with optional rotary positions: the forward
 * with its state record and the backward of both modes on views, e.g. q, k, v
 * read straight from a fused [B, N, 3, H, d] projection without copies.
 *
 * gla_fwd_framecausal_states_ex: gla_fwd_framecausal_states with q, k, v, g,
 * o as views (o may not overlap itself or any input) and rope as in
 * gla_fwd_framecausal_ex (the record then holds the turned-key states); the
 * workspace of gla_fwd_framecausal_workspace suffices.
 *
 * gla_bwd_framecausal_ex: the backward on views -- q, k, v, g, dO inputs; dq,
 * dk, dv, dg outputs, which may not overlap themselves, one another (each
 * view's span from its first to its last element counts, so gradients
 * interleaved in one fused buffer are refused with GLA_ERR_ALIAS), any input
 * or the workspace. states NULL: the states are recomputed (workspace
 * gla_bwd_framecausal_workspace); else the record written by
 * gla_fwd_framecausal_states(_ex) for the same inputs and rope (workspace
 * gla_bwd_framecausal_states_workspace). Without rope, results are bitwise
 * those of the contiguous calls on copies of the same tensors.
 *
 * gla_bwd_bidir_ex: the backward of gla_fwd_bidir_ex over N = F * T tokens
 * (the frames only place the rotary positions), views as above; workspace
 * gla_bwd_bidir_ex_workspace (that of gla_bwd_bidir for N without rope).
 *
 * Rotary positions (rope != NULL): the gradients of the rotary form of
 * gla_fwd_framecausal_ex / gla_fwd_bidir_ex (the chain rule through it: the
 * numerator's adjoints of phi(q) and phi(k) turn back by R^T before the
 * normaliser's terms are added). The matrix-core kernels take the turned
 * features as bf16 hi + lo pairs and the same table limit as the forward
 * (GLA_ERR_UNSUPPORTED beyond it). */
gla_status gla_fwd_framecausal_states_ex(const gla_tensor *q, const gla_tensor *k,
                                         const gla_tensor *v, const gla_tensor *g,
                                         const float *gamma, const float *S_in, const float *z_in,
                                         const gla_tensor *o, float *S_out, float *z_out,
                                         float *states, int B, int H, int F, int T, int d,
                                         gla_dtype dt, float eps, const gla_rope3d *rope,
                                         void *ws, size_t ws_bytes, void *stream);

gla_status gla_bwd_framecausal_ex(const gla_tensor *q, const gla_tensor *k, const gla_tensor *v,
                                  const gla_tensor *g, const float *gamma, const float *S_in,
                                  const float *z_in, const float *states, const gla_tensor *dO,
                                  const float *dS_out, const float *dz_out, const gla_tensor *dq,
                                  const gla_tensor *dk, const gla_tensor *dv,
                                  const gla_tensor *dg, float *dgamma, float *dS_in,
                                  float *dz_in, int B, int H, int F, int T, int d, gla_dtype dt,
                                  float eps, const gla_rope3d *rope, void *ws, size_t ws_bytes,
                                  void *stream);

size_t gla_bwd_bidir_ex_workspace(int B, int H, int F, int T, int d, const gla_rope3d *rope);

gla_status gla_bwd_bidir_ex(const gla_tensor *q, const gla_tensor *k, const gla_tensor *v,
                            const gla_tensor *g, const gla_tensor *dO, const gla_tensor *dq,
                            const gla_tensor *dk, const gla_tensor *dv, const gla_tensor *dg,
                            int B, int H, int F, int T, int d, gla_dtype dt, float eps,
                            const gla_rope3d *rope, void *ws, size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *gla_status_string(gla_status s);

/* Thread-local detail for the last non-OK status returned on this thread. */
const char *gla_last_error(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
int gla_version(void); /* 10600: gla_fwd_framecausal_noalloc (10500: rotary
                        positions in the training calls
                        (gla_fwd_framecausal_states_ex, gla_bwd_framecausal_ex take
                        rope) and gla_bwd_bidir_ex (10400: the two training calls on
                        views; 10300: the *_states calls; 10200: gla_softmax_anchor;
                        10100: the *_ex entry points)) */

/* ---- kernel timing for measurement tools ---------------------------------
 * Between gla_profile_begin and gla_profile_end, every kernel launched by the
 * entry points (on any stream, from any thread) is bracketed by a pair of HIP
 * events recorded on its stream. gla_profile_end waits for those events and
 * returns, per kernel kind ("kv", "carry", "readout", and for the backward
 * "bwd_q", "rev_scan", "bwd_k", "dgamma", and for the Gated DeltaNet "gdn_kv",
 * "gdn_scan", "gdn_readout"; "gdn_scan" includes the summing of a frame's parts
 * where the frame is split over several workgroups; and "anchor",
 * "anchor_redo"), the number of launches
 * and their summed event time. At most max_launches launches are timed; later
 * ones run untimed. Not meant to overlap with itself: one session at a time.
 * gla_profile_begin creates 2 * max_launches HIP events (max_launches must be
 * 1..65536, else GLA_ERR_VALUE); gla_profile_end destroys them. Returns
 * GLA_ERR_HIP if events cannot be created or read, GLA_ERR_VALUE if no session
 * is open. */
typedef struct gla_kernel_time {
  char name[16];
  int launches;
  double total_ms;
} gla_kernel_time;

gla_status gla_profile_begin(int max_launches);
gla_status gla_profile_end(gla_kernel_time *out, int max_out, int *n_out);

/* Launch log: with the environment variable GLA_LOG set to a nonzero integer
 * when the library first checks it, every call that launches kernels prints
 * one line with its plan (how the work is cut: kv parts P and frame groups G,
 * readout splits R, workgroups per kernel, workspace bytes) and one line per
 * launch, in order, to stderr, each starting "gla: ". */

/* Streaming bandwidth probe: one launch that moves `bytes` through HBM in the
 * access pattern of the mixer's kernels (16-byte loads and stores per lane,
 * whole 1 KiB runs per wave), for measuring the practical ceilings those
 * kernels are held against. kind: 0 read a, 1 read a nontemporal, 2 write
 * out, 3 write out nontemporal, 4 copy a to out, 5 the copy nontemporal,
 * 6 out = a ^ b (two reads and one write, the readout's pattern), 7 that
 * nontemporal, 8 a and b read nontemporally with plain stores of a ^ b into
 * one eighth of out (kv's pattern: two streamed reads with its frame states
 * written between them; every workgroup writes on one grid iteration in
 * eight). a, b, out: device buffers of `bytes` bytes each (as the kind
 * uses them; out is required for every kind: the read kinds may write a few
 * words into it), 16-byte aligned, out overlapping neither a nor b; `bytes` a
 * positive multiple of 256 KiB. Errors: GLA_ERR_VALUE (kind), GLA_ERR_SHAPE,
 * GLA_ERR_NULL, GLA_ERR_ALIGN, GLA_ERR_ALIAS, GLA_ERR_HIP (launch). */
gla_status gla_stream_probe(int kind, const void *a, const void *b, void *out, size_t bytes,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
