/*
 * hta.h -- C ABI of libhta: Hybrid Linear Temporal Attention on AMD MI355X (gfx950).
 *
 * The method (web pages on the Kairos world model, page "Kairos：面向物理 AI 的
 * 原生世界模型栈" on yingwang.github.io, section 二、方法, second pillar) mixes
 * three temporal attention branches over a frame-major token sequence:
 *   SWA  -- softmax attention restricted to a window of W frames (SWA paragraph);
 *   DSWA -- the same window counted in taps spaced `dilation` frames apart
 *           (DSWA paragraph, re-layout (B, F*L, D) -> (B*d, F/d*L, D));
 *   GLA  -- gated linear attention with the gated delta update of a fixed-size
 *           state S (GLA paragraph and its update equations);
 * and sums them into one mixed temporal representation (three-branch figure).
 *
 * Conventions shared by every entry point
 *   - Sequence tensors are contiguous [B][H][L][d], L = T*P, token t in frame t/P.
 *     q and k have d = dk, v and o have d = dv.
 *   - dtype HTA_BF16: q, k, v (and ring buffers) are bfloat16; accumulation,
 *     softmax, gates and the GLA state are fp32. dtype HTA_F32: everything fp32.
 *   - out_dtype: the dtype of o. HTA_F32 inputs give HTA_F32 outputs; HTA_BF16
 *     inputs may write o as HTA_F32 (the fp32 sum itself) or HTA_BF16 (that sum
 *     rounded once to nearest-even).
 *   - alpha, beta: fp32 [B][H][L], per-token forget gate alpha in (0, 1] and write
 *     strength beta in [0, 1] (the pages: beta = sigmoid(.), alpha in (0,1)).
 *   - GLA state: fp32 [B][H][dk][dv] holding S^T (S is dv x dk: v_old = S k).
 *   - Every pointer argument except `stream` (and the optional side stream and
 *     events in hta_params) is a DEVICE pointer owned by the caller. The library
 *     allocates no device memory and keeps no global state, with one exception:
 *     hta_stream_step_noalloc's fixed scratch array on each GPU and its address.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL =
 *     the null stream). Results are valid once the stream has synchronised.
 *   - All arguments are checked before anything is enqueued. On a non-zero
 *     status nothing has been enqueued and no output, state or ring is touched.
 *   - Outputs must not alias inputs. The state is updated in place.
 *   - Alignment: every sequence tensor (q, k, v, o, add, dout, dq, dk, dv, the
 *     projection's x, w, q, k, v), state, ring buffer, saved-activation block
 *     and workspace must start on a 16-byte boundary; alpha, beta, lse, dalpha
 *     and dbeta on a 4-byte boundary. Otherwise the call returns HTA_ERR_ALIGN.
 *     (Fresh torch or hipMalloc allocations are 256-byte aligned.)
 *   - Values: every finite input is supported, in either dtype. Some products of
 *     the bf16 paths run on fp16 operands; each such operand carries a power of
 *     two chosen from the data (per chunk, per state column group, or per tensor
 *     in the backward), an exact rescaling, so no range limit applies beyond
 *     fp32's. A NaN or Inf input makes every output that depends on it
 *     non-finite (in the GLA branch also the other tokens of its 64-token chunk,
 *     whose triangular products multiply masked entries by zero) and leaves the
 *     independent outputs as they would be without it.
 *   - Results are deterministic: identical calls return identical bits.
 *
 * Readings of the pages that the library implements (where they are silent):
 *   - the SWA window counts the current frame: frames f-W+1..f; attention is
 *     full inside a frame and never looks at later frames;
 *   - DSWA tap j reads frame f - j*dilation; taps before frame 0 are absent;
 *   - softmax scale 1/sqrt(dk) unless given;
 *   - GLA uses the GatedDeltaNet form the pages name as its basis:
 *       S_t = alpha_t * (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T,
 *       o_t = gla_scale * S_t q_t   (post-update state);
 *   - the hybrid output is the unweighted sum o_swa + o_dswa + o_gla in fp32,
 *     rounded once to the output dtype.
 */
#ifndef HTA_H
#define HTA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (int return value of every entry point). */
#define HTA_OK               0
#define HTA_ERR_NULL        (-1)  /* a required pointer is NULL                        */
#define HTA_ERR_SHAPE       (-2)  /* B,H,T,P < 1, or sizes overflow the index range    */
#define HTA_ERR_WINDOW      (-3)  /* window, taps or dilation < 1                      */
#define HTA_ERR_DTYPE       (-4)  /* dtype/out_dtype not HTA_F32 or HTA_BF16, or bf16 out of fp32 in */
#define HTA_ERR_UNSUPPORTED (-5)  /* dk/dv/chunk/taps outside the supported set        */
#define HTA_ERR_WORKSPACE   (-6)  /* workspace NULL or smaller than required           */
#define HTA_ERR_RING        (-7)  /* ring has fewer frames than the windows reach      */
#define HTA_ERR_HIP         (-8)  /* a HIP call failed; see hta_last_hip_error()       */
#define HTA_ERR_ALIAS       (-9)  /* an output overlaps an input                       */
#define HTA_ERR_ALIGN      (-10)  /* a device pointer is not aligned as required        */
#define HTA_ERR_SCRATCH    (-11)  /* needs more than HTA_NOALLOC_SCRATCH_BYTES          */

typedef enum { HTA_F32 = 0, HTA_BF16 = 1 } hta_dtype;

/* Supported sets: dk == dv in {64, 128}; HTA_BF16 requires dk == dv == 128.
 * gla_chunk in {16, 32, 64} for HTA_F32 and 64 for HTA_BF16.
 * window, taps <= 16; window, (taps-1)*dilation + 1 <= 4096 frames. */
typedef struct {
    int B, H;       /* batch, heads                                    */
    int T, P;       /* frames, tokens per frame (L = T*P)              */
    int dk, dv;     /* query/key and value head dims                   */
    int dtype;      /* hta_dtype of q, k, v and of the ring buffers    */
    int out_dtype;  /* hta_dtype of o (HTA_F32, or HTA_BF16 for bf16 inputs) */
} hta_shape;

typedef struct {
    int   swa_window;     /* W: SWA frames, current frame included          */
    int   dswa_taps;      /* W_d: DSWA taps (tap 0 is the current frame)    */
    int   dswa_dilation;  /* dilation between DSWA taps, in frames          */
    int   gla_chunk;      /* C: tokens per chunk of the chunked GLA         */
    float attn_scale;     /* softmax scale; 0 selects 1/sqrt(dk)            */
    float gla_scale;      /* GLA output scale; 0 selects 1                  */
    int   gla_form;       /* HTA_GLA_GATED_DELTA (0) or HTA_GLA_PRINTED (1) */
    /* Optional execution resources of the caller (all NULL: every launch goes on
     * the call's `stream`). side_stream: a second hipStream_t on the same device
     * on which the bf16 hybrid forward (and stream step, and training pair) runs
     * its attention work beside the GLA work on `stream`; fork_event, join_event:
     * two hipEvent_t the call records (on `stream`, resp. side_stream) and waits on,
     * both required with a side stream (HTA_ERR_NULL otherwise). The call orders
     * everything it enqueues on side_stream after the work already on `stream`,
     * and later work on `stream` after all of it. A call's use of the events must
     * not overlap another call's. The results are the same bits either way. The
     * overlap needs the two streams on different hardware queues: HIP deals its
     * streams out over a few queues in turn, and two streams that share one run
     * one after the other. */
    void* side_stream;
    void* fork_event;
    void* join_event;
} hta_params;

/*
 * GLA update forms (GLA paragraph and update equations of the Kairos page):
 *   HTA_GLA_GATED_DELTA -- the GatedDeltaNet update the page names as the basis:
 *       S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T;
 *   HTA_GLA_PRINTED     -- the three printed lines taken literally (v_old = S k,
 *       v_new = beta v + (1 - beta) v_old, S = alpha S - v_old k^T + v_new k^T),
 *       i.e. S_t = alpha_t S_{t-1} - beta_t (S_{t-1} k_t) k_t^T + beta_t v_t k_t^T:
 *       the forget gate does not scale the erase term.
 * Both give o_t = gla_scale * S_t q_t.
 */
#define HTA_GLA_GATED_DELTA 0
#define HTA_GLA_PRINTED     1

/* Operations whose workspace size hta_workspace_bytes() reports. */
#define HTA_OP_GLA          1
#define HTA_OP_HYBRID       2
#define HTA_OP_STREAM_STEP  3
#define HTA_OP_ATTN_BWD     4   /* hta_swa_bwd / hta_dswa_bwd (params may be NULL) */
#define HTA_OP_GLA_BWD      5   /* hta_gla_bwd (params: gla_chunk)                 */
#define HTA_OP_HYBRID_BWD   6   /* hta_hybrid_bwd                                  */
#define HTA_OP_SWA_DSWA     7   /* hta_swa_dswa_fwd_ex (params may be NULL)         */

/*
 * hta_workspace_bytes -- device workspace (bytes, 256-byte aligned start
 * expected) that `op` needs for `shape`/`params`. For HTA_OP_STREAM_STEP pass
 * the per-frame shape (T = 1). Returns 0 if the arguments are invalid (an op
 * that needs no workspace also returns 0 with valid arguments: HTA_OP_*
 * always needs some, so 0 means invalid).
 */
size_t hta_workspace_bytes(int op, const hta_shape* shape, const hta_params* params);

/*
 * hta_swa_fwd -- SWA branch alone (SWA paragraph): o[t] = softmax attention of
 * q[t] over every key of frames f-window+1 .. f (>= 0), f = t / P.
 * q, k: [B][H][L][dk]; v, o: [B][H][L][dv]; scale 0 selects 1/sqrt(dk).
 */
int hta_swa_fwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                void* o, int window_frames, float scale, void* stream);

/*
 * hta_dswa_fwd -- DSWA branch alone (DSWA paragraph): o[t] = softmax attention
 * of q[t] over every key of frames f - j*dilation, 0 <= j < taps, >= 0.
 */
int hta_dswa_fwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                 void* o, int taps, int dilation_frames, float scale, void* stream);

/*
 * hta_swa_fwd_lse / hta_dswa_fwd_lse -- hta_swa_fwd / hta_dswa_fwd that also
 * write, for the backward pass, lse: fp32 [B][H][L] with
 *   lse[t] = log sum_s exp(scale * q_t . k_s)   (natural log)
 * over the keys s of row t's window. lse must not overlap q, k, v or o.
 */
int hta_swa_fwd_lse(const hta_shape* shape, const void* q, const void* k, const void* v,
                    void* o, float* lse, int window_frames, float scale, void* stream);
int hta_dswa_fwd_lse(const hta_shape* shape, const void* q, const void* k, const void* v,
                     void* o, float* lse, int taps, int dilation_frames, float scale,
                     void* stream);

/*
 * hta_swa_bwd / hta_dswa_bwd -- gradient of one attention branch (the SWA or
 * DSWA paragraph's forward), by the chain rule through softmax:
 *   p_ts = exp(scale q_t.k_s - lse_t),  D_t = dout_t . o_t,
 *   ds_ts = p_ts (dout_t . v_s - D_t),
 *   dq_t = scale sum_s ds_ts k_s,  dk_s = scale sum_t ds_ts q_t,  dv_s = sum_t p_ts dout_t.
 * Inputs: q, k, v as in the forward (dtype); o and lse from hta_*_fwd_lse with
 * the same window and scale; dout = dL/do, [B][H][L][dv] in out_dtype (the
 * dtype of o). Outputs dq, dk ([B][H][L][dk]) and dv ([B][H][L][dv]) in dtype,
 * each written once (not accumulated). With bf16 inputs the products run on
 * bf16 MFMA with fp32 accumulation: p and ds are rounded to bf16 as operands,
 * dout is rounded to bf16 (and D taken from the rounded values).
 * workspace: >= hta_workspace_bytes(HTA_OP_ATTN_BWD, shape, NULL). Outputs
 * must not overlap the inputs, each other or the workspace.
 */
int hta_swa_bwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                const void* o, const float* lse, const void* dout, void* dq, void* dk,
                void* dv, int window_frames, float scale, void* workspace,
                size_t workspace_bytes, void* stream);
int hta_dswa_bwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* dout, void* dq, void* dk,
                 void* dv, int taps, int dilation_frames, float scale, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * hta_swa_dswa_fwd -- SWA and DSWA summed: o = o_swa + o_dswa (+ add). The
 * branches run as two passes accumulating in fp32 (in o when out_dtype is
 * HTA_F32, else in `add`); a bf16 o with add == NULL is computed in one fused
 * pass instead. params: swa_window, dswa_taps, dswa_dilation,
 * attn_scale (gla_* ignored). add: NULL, or an fp32 [B][H][L][dv] partial
 * (e.g. the GLA branch) added before the single rounding to out_dtype; add
 * may equal o when out_dtype is HTA_F32 (in-place accumulation), and must not
 * overlap q, k or v otherwise.
 */
int hta_swa_dswa_fwd(const hta_shape* shape, const hta_params* params,
                     const void* q, const void* k, const void* v, const float* add,
                     void* o, void* stream);

/*
 * hta_swa_dswa_fwd_ex -- hta_swa_dswa_fwd computed in ONE pass over the tap
 * frames with bf16 inputs: the query's own frame, common to both windows, is
 * attended once; its softmax state is kept in the workspace while the SWA taps
 * finish (that branch's output goes to o, or to the workspace), then resumed for
 * the DSWA taps, and the epilogue adds the two branches (and `add`). Same
 * arguments, results and aliasing rules as hta_swa_dswa_fwd, plus
 * workspace >= hta_workspace_bytes(HTA_OP_SWA_DSWA, shape, NULL) not overlapping
 * any other argument. fp32 inputs behave exactly as hta_swa_dswa_fwd.
 */
int hta_swa_dswa_fwd_ex(const hta_shape* shape, const hta_params* params,
                        const void* q, const void* k, const void* v, const float* add,
                        void* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * hta_gla_fwd -- GLA branch alone (GLA paragraph and update equations), chunked.
 * state: fp32 [B][H][dk][dv] = S^T; in: initial state (zero it for S_0 = 0),
 * out: state after the last token. o: [B][H][L][dv] (o_t = scale * S_t q_t).
 * workspace: >= hta_workspace_bytes(HTA_OP_GLA, shape, params with gla_chunk).
 */
int hta_gla_fwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                const float* alpha, const float* beta, float* state, void* o,
                int chunk, float scale, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * hta_gla_fwd_ex -- hta_gla_fwd with the chunk, the output scale and the update
 * form taken from params (gla_chunk, gla_scale, gla_form; the attention fields
 * are ignored). Same buffers, workspace and error behaviour as hta_gla_fwd;
 * HTA_ERR_UNSUPPORTED for a gla_form other than the two above.
 */
int hta_gla_fwd_ex(const hta_shape* shape, const hta_params* params,
                   const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, float* state, void* o,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * hta_gla_bwd -- gradient of the GLA branch (GLA paragraph and update equations;
 * form, chunk and output scale from params as in hta_gla_fwd_ex). With the
 * state M = S^T, the forward maps (q, k, v, alpha, beta, M_0) to (o, M_L); this
 * call returns the vector-Jacobian product for dL/do and dL/dM_L:
 *   state0: fp32 [B][H][dk][dv], the initial state M_0 the forward started from
 *           (zeros for S_0 = 0); not modified.
 *   dout:   dL/do, [B][H][L][dv] in out_dtype.
 *   dstate: fp32 [B][H][dk][dv], in: dL/dM_L (zero it when the loss does not
 *           read the final state), out: dL/dM_0.
 *   dq, dk ([B][H][L][dk]), dv ([B][H][L][dv]) in dtype; dalpha, dbeta fp32
 *           [B][H][L]; each written once.
 * The forward is recomputed inside the call from the inputs and state0. The
 * gradient with respect to alpha goes through log(alpha): alpha must be > 0.
 * workspace: >= hta_workspace_bytes(HTA_OP_GLA_BWD, shape, params). Outputs must
 * not overlap the inputs, each other or the workspace.
 */
int hta_gla_bwd(const hta_shape* shape, const hta_params* params,
                const void* q, const void* k, const void* v,
                const float* alpha, const float* beta, const float* state0,
                const void* dout, float* dstate, void* dq, void* dk, void* dv,
                float* dalpha, float* dbeta, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * hta_hybrid_fwd -- the whole layer (three-branch figure): o = o_swa + o_dswa + o_gla
 * with shared q, k, v; the GLA branch in params->gla_form. state as in hta_gla_fwd. workspace: >=
 * hta_workspace_bytes(HTA_OP_HYBRID, shape, params).
 * bf16 inputs: the GLA branch goes into an fp32 partial in the workspace; one
 * attention pass runs both windows (as in hta_swa_dswa_fwd_ex). Without a side
 * stream in params, the GLA branch runs first and the pass adds its partial in
 * its epilogue. With one, the pass runs on the side stream beside the GLA chunk
 * scan on `stream`, and after the join one elementwise kernel adds the partial.
 * Either way o is (DSWA + SWA) + GLA in fp32, rounded once: the same bits.
 * fp32 inputs: GLA into o, then SWA + DSWA adding it, all on `stream`.
 */
int hta_hybrid_fwd(const hta_shape* shape, const hta_params* params,
                   const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, float* state, void* o,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training: hta_hybrid_fwd_train is hta_hybrid_fwd (same arguments, workspace
 * of HTA_OP_HYBRID, same stream behaviour) that also fills `saved`, a caller
 * buffer of hta_hybrid_saved_bytes(shape) bytes (0 on an invalid shape), with
 * what the backward pass needs: the initial GLA state (copied before the call
 * advances `state`), each attention branch's own output (fp32) and per-row
 * log-sum-exp. `saved` must not overlap any other argument.
 *
 * hta_hybrid_bwd -- gradient of the whole layer, o = o_swa + o_dswa + o_gla, for
 * dout = dL/do ([B][H][L][dv], out_dtype) and dstate = dL/dM_L (in; zero it if
 * the loss does not read the final state), from the inputs of the forward and
 * its `saved` buffer. Writes dq, dk, dv (dtype; the three branches' gradients
 * summed in fp32 and rounded once), dalpha, dbeta (fp32 [B][H][L]) and dstate
 * (out: dL/dM_0). The GLA branch's forward is recomputed inside the call. The
 * same numerics as hta_swa_bwd / hta_dswa_bwd and hta_gla_bwd apply.
 * workspace: >= hta_workspace_bytes(HTA_OP_HYBRID_BWD, shape, params). Outputs
 * must not overlap the inputs, each other or the workspace.
 */
size_t hta_hybrid_saved_bytes(const hta_shape* shape);
int hta_hybrid_fwd_train(const hta_shape* shape, const hta_params* params,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, float* state, void* o,
                         void* saved, void* workspace, size_t workspace_bytes, void* stream);
int hta_hybrid_bwd(const hta_shape* shape, const hta_params* params,
                   const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const void* saved,
                   const void* dout, float* dstate, void* dq, void* dk, void* dv,
                   float* dalpha, float* dbeta, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Streaming context: the complete resumable memory of the layer after
 * n_frames frames -- the last R frames of K and V in a ring (frame n lives in
 * slot n mod R) and the GLA state. The caller owns every buffer; copying the
 * three buffers and n_frames checkpoints the stream exactly.
 */
typedef struct {
    hta_shape  s;          /* T is ignored (one frame per step); P = tokens per frame */
    hta_params p;
    int        R;          /* ring frames; must be >= max(W, (W_d - 1) * dil + 1)     */
    void*      ring_k;     /* [B][H][R][P][dk], dtype s.dtype                          */
    void*      ring_v;     /* [B][H][R][P][dv]                                         */
    float*     state;      /* [B][H][dk][dv] fp32, S^T                                 */
    long long  n_frames;   /* frames committed so far                                  */
} hta_stream_ctx;

/*
 * hta_stream_init -- start a stream after a prefix of T_prefix frames.
 * k_prefix, v_prefix: [B][H][T_prefix*P][d] (may be NULL when T_prefix == 0);
 * the last min(T_prefix, R) frames are copied into their ring slots.
 * state_prefix: the GLA state after the prefix (e.g. hta_hybrid_fwd's output
 * state), copied into ctx->state; NULL sets the state to zero.
 * Sets ctx->n_frames = T_prefix on success.
 */
int hta_stream_init(hta_stream_ctx* ctx, const void* k_prefix, const void* v_prefix,
                    int T_prefix, const float* state_prefix, void* stream);

/*
 * hta_stream_step -- append one frame n = ctx->n_frames:
 *   1. its K and V go to ring slot n mod R;
 *   2. the GLA state advances over its P tokens (chunks start at the frame);
 *   3. if o != NULL, o = o_swa + o_dswa + o_gla for the frame's P queries, with
 *      SWA over frames n..n-W+1 and DSWA over n - j*dil, read from the ring.
 * q, k, v: [B][H][P][d]; alpha, beta: [B][H][P]; o: [B][H][P][dv] or NULL
 * (commit only). workspace: >= hta_workspace_bytes(HTA_OP_STREAM_STEP,
 * &ctx->s with T = 1, &ctx->p). With bf16 inputs and o != NULL, steps 2 and 3
 * run as in hta_hybrid_fwd (beside each other when ctx->p carries a side
 * stream). ctx->n_frames is incremented after a successful enqueue. A context
 * must not be used by two threads at once.
 */
int hta_stream_step(hta_stream_ctx* ctx, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, void* o,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * hta_stream_step_noalloc -- hta_stream_step without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * results (the same kernels, bit for bit), context update and error behaviour
 * as hta_stream_step, which it calls with the library's scratch instead of a
 * caller workspace. The scratch is one fixed array of HTA_NOALLOC_SCRATCH_BYTES
 * per GPU inside the library, allocated when the library's code loads on that
 * GPU and held until the process ends; this call allocates and frees nothing.
 *   - Returns HTA_ERR_SCRATCH (nothing enqueued) when the step needs more than
 *     HTA_NOALLOC_SCRATCH_BYTES, i.e. when hta_workspace_bytes(HTA_OP_STREAM_STEP,
 *     ...) (or its commit-only share) exceeds it. 128 MiB holds B*H = 32 heads
 *     of P = 1560 tokens with bf16 inputs and either output dtype.
 *   - `stream` must belong to the current device (HTA_ERR_UNSUPPORTED otherwise).
 *   - Every call on a GPU uses that GPU's one array: calls whose work overlaps
 *     on one GPU (other streams, other threads, other contexts) race and give
 *     undefined results. Serialise them, e.g. on one stream. The array keeps the
 *     last call's contents; the step writes each scratch byte before reading it.
 *   - The first call on a device looks up the array's address there (a HIP
 *     symbol query, no allocation); later calls reuse it.
 */
#define HTA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int hta_stream_step_noalloc(hta_stream_ctx* ctx, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, void* o, void* stream);

/*
 * hta_project_fwd -- the input side of the GLA branch (GLA paragraph: q = W_Q x,
 * k = W_K x, v = W_V x, beta = sigmoid(W_beta x), and a forget gate in (0, 1)
 * computed from the input, read as alpha = sigmoid(W_alpha x)), for every
 * token at once, in the layouts the other entry points take.
 *   shape: B, H, T, P (L = T*P tokens per sequence), dk = dv = 128, dtype
 *          HTA_BF16 (out_dtype ignored); H a multiple of 4 with 2H <= 128.
 *   x:     [B][L][d_model] bf16 token features, d_model a multiple of 64.
 *   w:     [d_model][N] bf16, N = 3*H*128 + 2*H; columns q heads 0..H-1, then k
 *          heads, v heads, H alpha columns, H beta columns.
 *   q, k, v: [B][H][L][128] bf16 outputs; alpha, beta: [B][H][L] fp32.
 *   flags: HTA_NORM_Q and / or HTA_NORM_K L2-normalise q / k per token and
 *          head (a zero vector stays zero).
 * fp32 accumulation; each output rounded once. Outputs must not overlap the
 * inputs or each other. HTA_ERR_UNSUPPORTED for other dtypes, head dims,
 * head counts or model widths.
 */
#define HTA_NORM_Q 1
#define HTA_NORM_K 2
int hta_project_fwd(const hta_shape* shape, int d_model, const void* x, const void* w,
                    void* q, void* k, void* v, float* alpha, float* beta, int flags,
                    void* stream);

/* Human-readable name of a status code (static string). */
const char* hta_status_string(int status);

/* hipError_t of the last HTA_ERR_HIP returned on the calling thread (0 if none). */
int hta_last_hip_error(void);

/* Library version, e.g. "hta 0.1.0 gfx950". */
const char* hta_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HTA_H */
