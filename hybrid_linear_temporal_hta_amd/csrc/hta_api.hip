// hta_api.hip -- the C ABI of libhta (declared in include/hta.h): argument
// validation, workspace layout and the order of kernel launches.
//
// The branches and their sum follow page "Kairos：面向物理 AI 的原生世界模型栈"
// (yingwang.github.io), section 二、方法, second pillar: SWA, DSWA and GLA
// paragraphs and the three-branch figure. Every check runs before the first
// launch, so a failing call enqueues nothing and touches no output.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/hta.h"
#include "hta_internal.h"


namespace {

thread_local int g_last_hip_error = 0;

constexpr long long kMaxElems = (1LL << 62);
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dtype) { return dtype == HTA_BF16 ? 2 : 4; }

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return HTA_ERR_HIP;
}

struct Range {
    uintptr_t lo, hi;
};

Range range_of(const void* p, size_t bytes) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Sequence tensors, states, rings, saved activations and workspaces are read and
// written 16 bytes at a time (mask 15); per-token gates and statistics one float
// at a time (mask 3). NULL pointers pass.
template <typename... P>
int check_align(uintptr_t mask, const P*... p) {
    uintptr_t bits = 0;
    ((bits |= reinterpret_cast<uintptr_t>(p)), ...);
    return (bits & mask) ? HTA_ERR_ALIGN : HTA_OK;
}

// Shape checks shared by every entry point. L = T*P.
int check_shape(const hta_shape* s) {
    if (!s) return HTA_ERR_NULL;
    if (s->dtype != HTA_F32 && s->dtype != HTA_BF16) return HTA_ERR_DTYPE;
    if (s->out_dtype != HTA_F32 && s->out_dtype != HTA_BF16) return HTA_ERR_DTYPE;
    if (s->dtype == HTA_F32 && s->out_dtype != HTA_F32) return HTA_ERR_DTYPE;
    if (s->B < 1 || s->H < 1 || s->T < 1 || s->P < 1 || s->dk < 1 || s->dv < 1) return HTA_ERR_SHAPE;
    if (s->dk != s->dv) return HTA_ERR_UNSUPPORTED;
    if (s->dk != 64 && s->dk != 128) return HTA_ERR_UNSUPPORTED;
    if (s->dtype == HTA_BF16 && s->dk != 128) return HTA_ERR_UNSUPPORTED;
    const long long L = (long long)s->T * s->P;
    const long long bh = (long long)s->B * s->H;
    if (bh > (1LL << 30) || L > (1LL << 40)) return HTA_ERR_SHAPE;
    if ((double)bh * (double)L * (double)s->dk >= (double)kMaxElems) return HTA_ERR_SHAPE;
    if (bh * (long long)((s->P + 63) / 64) * s->T > 0x7fffffffLL) return HTA_ERR_SHAPE;
    return HTA_OK;
}

int check_scale(float scale) {
    if (!(scale >= 0.f) || !isfinite(scale)) return HTA_ERR_UNSUPPORTED;
    return HTA_OK;
}

int check_window(int window) { return (window >= 1 && window <= hta::kMaxTaps) ? HTA_OK : HTA_ERR_WINDOW; }

int check_dilated(int taps, int dil) {
    if (taps < 1 || taps > hta::kMaxTaps || dil < 1) return HTA_ERR_WINDOW;
    if ((long long)(taps - 1) * dil + 1 > 4096) return HTA_ERR_WINDOW;
    return HTA_OK;
}

int check_chunk(int dtype, int chunk) {
    if (dtype == HTA_BF16) return chunk == 64 ? HTA_OK : HTA_ERR_UNSUPPORTED;
    return (chunk == 16 || chunk == 32 || chunk == 64) ? HTA_OK : HTA_ERR_UNSUPPORTED;
}

int check_params(const hta_shape* s, const hta_params* p) {
    if (!p) return HTA_ERR_NULL;
    int st;
    if ((st = check_window(p->swa_window)) != HTA_OK) return st;
    if ((st = check_dilated(p->dswa_taps, p->dswa_dilation)) != HTA_OK) return st;
    if ((st = check_chunk(s->dtype, p->gla_chunk)) != HTA_OK) return st;
    if ((st = check_scale(p->attn_scale)) != HTA_OK) return st;
    if (!isfinite(p->gla_scale)) return HTA_ERR_UNSUPPORTED;
    if (p->gla_form != HTA_GLA_GATED_DELTA && p->gla_form != HTA_GLA_PRINTED)
        return HTA_ERR_UNSUPPORTED;
    if (p->side_stream && (!p->fork_event || !p->join_event)) return HTA_ERR_NULL;
    return HTA_OK;
}

float attn_scale_of(float scale, int dk) { return scale > 0.f ? scale : 1.0f / sqrtf((float)dk); }
float gla_scale_of(float scale) { return scale != 0.f ? scale : 1.0f; }

size_t seq_bytes(const hta_shape* s, int d) {
    return (size_t)s->B * s->H * (size_t)s->T * s->P * d * elem_bytes(s->dtype);
}
size_t out_bytes(const hta_shape* s) {
    return (size_t)s->B * s->H * (size_t)s->T * s->P * s->dv * elem_bytes(s->out_dtype);
}
size_t gate_bytes(const hta_shape* s) { return (size_t)s->B * s->H * (size_t)s->T * s->P * 4; }
size_t state_bytes(const hta_shape* s) { return (size_t)s->B * s->H * s->dk * s->dv * 4; }

// Workspace of the bf16 hybrid and stream step: [GLA chunk blocks][fp32 GLA
// partial][fp32 SWA output (bf16 o only)][parked softmax states].
size_t gla_ws(const hta_shape* s, int chunk) {
    (void)chunk;
    if (s->dtype == HTA_F32) return kAlign;
    const long long L = (long long)s->T * s->P;
    return align_up(hta::gla_fwd_workspace_bytes(s->B * s->H, L));
}
size_t fp32_seq_bytes(const hta_shape* s) {
    return align_up((size_t)s->B * s->H * (size_t)s->T * s->P * s->dv * 4);
}
size_t park_ws(const hta_shape* s) {
    return align_up(hta::win_attn_park_bytes(s->B * s->H, s->T, s->P));
}
// bf16 inputs: the GLA branch runs first into an fp32 partial; the one-pass
// attention then adds it in its epilogue. The SWA branch's output (written at the
// switch between the windows) goes to o itself when o is fp32, else to an fp32
// buffer. fp32 inputs (small workloads) keep the GLA partial in o.
size_t partial_ws(const hta_shape* s) {
    if (s->dtype == HTA_F32) return 0;
    return fp32_seq_bytes(s) * (s->out_dtype == HTA_F32 ? 1 : 2) + park_ws(s);
}
struct Partials {
    float* gla;    // fp32 GLA partial
    float* oa;     // fp32 SWA output (o itself when o is fp32)
    float* park;   // parked softmax states
};
Partials partials_of(const hta_shape* s, char* partials, void* o) {
    Partials pt;
    pt.gla = reinterpret_cast<float*>(partials);
    char* c = partials + fp32_seq_bytes(s);
    if (s->out_dtype == HTA_F32) {
        pt.oa = static_cast<float*>(o);
    } else {
        pt.oa = reinterpret_cast<float*>(c);
        c += fp32_seq_bytes(s);
    }
    pt.park = reinterpret_cast<float*>(c);
    return pt;
}

// The caller's side stream (hta_params): work that runs beside `stream`, forked
// and joined through the caller's two events. NULL: everything on `stream`.
struct Side {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
Side side_of(const hta_params* p) {
    Side d;
    if (p && p->side_stream) {
        d.s = static_cast<hipStream_t>(p->side_stream);
        d.fork = static_cast<hipEvent_t>(p->fork_event);
        d.join = static_cast<hipEvent_t>(p->join_event);
    }
    return d;
}
// Work enqueued on d.s after fork() is ordered after everything already on sm;
// join() orders later work on sm after everything enqueued on d.s.
hipError_t fork(const Side& d, hipStream_t sm) {
    hipError_t e = hipEventRecord(d.fork, sm);
    return e == hipSuccess ? hipStreamWaitEvent(d.s, d.fork, 0) : e;
}
hipError_t join(const Side& d, hipStream_t sm) {
    hipError_t e = hipEventRecord(d.join, d.s);
    return e == hipSuccess ? hipStreamWaitEvent(sm, d.join, 0) : e;
}

hta::WinLaunch win_base(const hta_shape* s, const void* q, const void* k, const void* v, void* o,
                        float scale) {
    hta::WinLaunch w;
    memset(&w, 0, sizeof(w));
    const long long L = (long long)s->T * s->P;
    w.q = q; w.k = k; w.v = v; w.o = o; w.add = nullptr;
    w.q_bh = L * s->dk;
    w.kv_bh = L * s->dk;
    w.kv_frame = (long long)s->P * s->dk;
    w.BH = s->B * s->H;
    w.P = s->P;
    w.Tq = s->T;
    w.frame0 = 0;
    w.R = 0;
    w.scale = attn_scale_of(scale, s->dk);
    w.d = s->dk;
    w.dtype = s->dtype;
    w.out_f32 = s->out_dtype == HTA_F32 ? 1 : 0;
    return w;
}

void taps_swa(hta::WinTaps& t, int window) {
    t.nA = window;
    for (int j = 0; j < window; ++j) t.offA[j] = j;
    t.nB = 0;
}

void taps_dswa(hta::WinTaps& t, int taps, int dil) {
    t.nA = taps;
    for (int j = 0; j < taps; ++j) t.offA[j] = j * dil;
    t.nB = 0;
}

// SWA as branch A (own frame first), DSWA taps 1.. as branch B.
void taps_hybrid(hta::WinTaps& t, int window, int taps, int dil) {
    t.nA = window;
    for (int j = 0; j < window; ++j) t.offA[j] = j;
    t.nB = taps - 1;
    for (int j = 1; j < taps; ++j) t.offB[j - 1] = j * dil;
}

// SWA + DSWA (+ w.add) into w.o without a workspace (hta_swa_dswa_fwd, the fp32
// hybrid and stream paths; the bf16 hybrid runs the one-pass kernel, which
// parks state in a workspace). Split: an SWA pass into an fp32 buffer (o itself,
// or the caller's fp32 partial), then a DSWA pass adding it; each pass keeps one
// accumulator set and runs at two waves per SIMD. With a bf16 o and no fp32
// partial to accumulate in: one pass with two accumulator sets (one wave per
// SIMD), which rounds the sum once without an intermediate buffer.
hipError_t run_swa_dswa(hta::WinLaunch w, int window, int taps, int dil, hipStream_t st) {
    if (w.dtype != HTA_BF16 || (!w.out_f32 && !w.add)) {
        w.nbr = 2;
        taps_hybrid(w.taps, window, taps, dil);
        return hta::launch_win_attn(w, st);
    }
    hta::WinLaunch a = w;
    a.nbr = 1;
    taps_swa(a.taps, window);
    float* mid = w.out_f32 ? static_cast<float*>(w.o) : const_cast<float*>(w.add);
    a.o = mid;
    a.out_f32 = 1;
    hipError_t e = hta::launch_win_attn(a, st);
    if (e != hipSuccess) return e;
    hta::WinLaunch b = w;
    b.nbr = 1;
    taps_dswa(b.taps, taps, dil);
    b.add = mid;
    return hta::launch_win_attn(b, st);
}

hta::GlaLaunch gla_base(const hta_shape* s, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, float* state, void* o,
                        int chunk, float scale, void* ws, size_t ws_bytes, int form = 0) {
    hta::GlaLaunch g;
    memset(&g, 0, sizeof(g));
    g.q = q; g.k = k; g.v = v; g.alpha = alpha; g.beta = beta; g.state = state; g.o = o;
    g.out_f32 = s->out_dtype == HTA_F32 ? 1 : 0;
    g.L = (long long)s->T * s->P;
    g.BH = s->B * s->H;
    g.d = s->dk;
    g.chunk = chunk;
    g.scale = gla_scale_of(scale);
    g.dtype = s->dtype;
    g.ws = ws;
    g.ws_bytes = ws_bytes;
    g.form = form;
    return g;
}

hipError_t run_gla(const hta::GlaLaunch& g, hipStream_t st) {
    return g.dtype == HTA_F32 ? hta::launch_gla_f32(g, st) : hta::launch_gla_fwd(g, st);
}

size_t gla_bwd_ws(const hta_shape* s) {
    return align_up(hta::gla_bwd_workspace_bytes(s->dtype, s->B * s->H, (long long)s->T * s->P,
                                                 s->dk));
}

hta::GlaBwdLaunch gla_bwd_base(const hta_shape* s, const hta_params* p, const void* q,
                               const void* k, const void* v, const float* alpha,
                               const float* beta, const float* state0, const void* dout,
                               float* dstate, void* dq, void* dk, void* dv, float* dalpha,
                               float* dbeta, void* ws, size_t ws_bytes) {
    hta::GlaBwdLaunch b;
    memset(&b, 0, sizeof(b));
    b.q = q; b.k = k; b.v = v; b.alpha = alpha; b.beta = beta; b.state0 = state0;
    b.dout = dout;
    b.do_f32 = s->out_dtype == HTA_F32 ? 1 : 0;
    b.dstate = dstate;
    b.dq = dq; b.dk = dk; b.dv = dv; b.dalpha = dalpha; b.dbeta = dbeta;
    b.L = (long long)s->T * s->P;
    b.BH = s->B * s->H;
    b.d = s->dk;
    b.chunk = p->gla_chunk;
    b.scale = gla_scale_of(p->gla_scale);
    b.dtype = s->dtype;
    b.form = p->gla_form;
    b.ws = ws;
    b.ws_bytes = ws_bytes;
    return b;
}

// Training outputs of the attention pass (all optional): each branch's
// log-sum-exp, and the DSWA branch's own output.
struct TrainOut {
    float* lse_a = nullptr;
    float* lse_b = nullptr;
    float* obr_b = nullptr;
};

// hta_swa_dswa_fwd_ex workspace: [park][fp32 branch-A output]; fp32 inputs need none.
size_t swa_dswa_ws(const hta_shape* s) {
    if (s->dtype != HTA_BF16) return kAlign;
    return park_ws(s) + fp32_seq_bytes(s);
}

// bf16 hybrid (and streamed frame). One attention pass runs both windows with one
// accumulator set (the query's own frame, common to both, is attended once: its
// softmax state is parked in memory while the SWA taps finish, then resumed for
// the DSWA taps); the GLA branch (chunk-parallel prep, then the chunk scan) goes
// into an fp32 partial.
//   - Without a side stream, on `sm` in order: the GLA branch over the whole chip,
//     then the attention pass, whose epilogue adds both windows and the GLA
//     partial and rounds once.
//   - With the caller's side stream: the GLA prep on `sm`, then the attention pass
//     (its sum in fp32, no partial) on the side stream beside the GLA scan on `sm`
//     in its narrow shape (two workgroups per head, so the pass keeps nearly the
//     whole chip); after the join one elementwise pass adds the GLA partial and
//     rounds once. Both routes form (DSWA + SWA) + GLA in fp32 in the same order,
//     so they give the same bits.
// For a training forward, `tr` receives each branch's log-sum-exp and branch B's
// (DSWA's) output, and `oa` (when given) branch A's (SWA's) output.
hipError_t run_hybrid(hta::GlaLaunch g, const hta::WinLaunch& w, const Partials& pt,
                      const hta_params* p, hipStream_t sm, const TrainOut& tr = TrainOut(),
                      float* oa = nullptr) {
    g.o = pt.gla;
    g.out_f32 = 1;
    hta::WinLaunch f = w;
    f.nbr = 3;
    taps_hybrid(f.taps, p->swa_window, p->dswa_taps, p->dswa_dilation);
    f.oa = oa ? oa : pt.oa;
    f.park = pt.park;
    f.add2 = nullptr;
    f.lse = tr.lse_a;
    f.lse2 = tr.lse_b;
    f.obr = tr.obr_b;
    const Side d = side_of(p);
    hipError_t e;
    if (!d.s) {
        if ((e = hta::launch_gla_fwd(g, sm)) != hipSuccess) return e;
        f.add = pt.gla;
        return hta::launch_win_attn(f, sm);
    }
    // the pass's fp32 sum: o itself, or the SWA buffer (read back in place, row by row)
    float* att = w.out_f32 ? static_cast<float*>(w.o) : pt.oa;
    f.o = att;
    f.out_f32 = 1;
    f.add = nullptr;
    // prep first (it needs the whole chip briefly), then the scan on a few CUs
    // beside the attention pass (started at once, the attention holds every
    // CU's LDS and the scan's workgroups could not be placed until it drained)
    if ((e = hta::launch_gla_fwd(g, sm, hta::kGlaPrep)) != hipSuccess) return e;
    if ((e = fork(d, sm)) != hipSuccess) return e;
    if ((e = hta::launch_gla_fwd(g, sm, hta::kGlaScanNarrow)) != hipSuccess) return e;
    if ((e = hta::launch_win_attn(f, d.s)) != hipSuccess) return e;
    if ((e = join(d, sm)) != hipSuccess) return e;
    const long long n = (long long)w.BH * w.Tq * w.P * w.d;
    return hta::launch_add_f32(w.o, w.out_f32 ? 0 : 1, att, pt.gla, n, sm);
}

// What a training forward keeps for hta_hybrid_bwd (caller-owned `saved`).
struct Saved {
    float* o_swa;      // [BH][L][dv] the SWA branch's output
    float* o_dswa;     // [BH][L][dv] the DSWA branch's output
    float* lse_swa;    // [BH][L]
    float* lse_dswa;   // [BH][L]
    float* state0;     // [BH][dk][dv] the initial GLA state
};
size_t saved_bytes(const hta_shape* s) {
    return 2 * fp32_seq_bytes(s) + 2 * align_up(gate_bytes(s)) + align_up(state_bytes(s));
}
Saved saved_of(const hta_shape* s, void* p) {
    char* c = static_cast<char*>(p);
    Saved v;
    v.o_swa = reinterpret_cast<float*>(c); c += fp32_seq_bytes(s);
    v.o_dswa = reinterpret_cast<float*>(c); c += fp32_seq_bytes(s);
    v.lse_swa = reinterpret_cast<float*>(c); c += align_up(gate_bytes(s));
    v.lse_dswa = reinterpret_cast<float*>(c); c += align_up(gate_bytes(s));
    v.state0 = reinterpret_cast<float*>(c);
    return v;
}



// Backward of one attention branch. Workspace: per-row stats {lse log2(e), D}
// with 64 rows of padding (the key pass stages 64-row tiles of it), then, for
// bf16 inputs with an fp32 dout, dout rounded to bf16.
size_t attn_bwd_stats_bytes(const hta_shape* s) {
    return align_up(((size_t)s->B * s->H * (size_t)s->T * s->P + 64) * 8);
}
// bf16 inputs: the maxima that scale dS and the fp16 copies (256 bytes: |dO|, |v|,
// |q|, |k|) and the fp16 copies of q and k.
size_t attn_bwd_aux_bytes(const hta_shape* s) {
    if (s->dtype != HTA_BF16) return 0;
    return kAlign + 2 * align_up((size_t)s->B * s->H * (size_t)s->T * s->P * s->dk * 2);
}
size_t do_copy_bytes(const hta_shape* s) {
    if (s->dtype == HTA_BF16 && s->out_dtype == HTA_F32)
        return align_up((size_t)s->B * s->H * (size_t)s->T * s->P * s->dv * 2);
    return 0;
}
size_t attn_bwd_ws(const hta_shape* s) {
    return attn_bwd_stats_bytes(s) + attn_bwd_aux_bytes(s) + do_copy_bytes(s);
}

// Points the prep and the passes at the aux region (bf16): maxima, q16, k16;
// zeroes the maxima (a kernel, not a memset).
hipError_t bind_bwd_aux(const hta_shape* s, char* aux, hta::BwdPrep& p, hipStream_t st) {
    if (s->dtype != HTA_BF16) return hipSuccess;
    const size_t nqk = align_up((size_t)s->B * s->H * (size_t)s->T * s->P * s->dk * 2);
    p.gmax = reinterpret_cast<unsigned*>(aux);
    p.q16 = aux + kAlign;
    p.k16 = aux + kAlign + nqk;
    return hta::launch_fill_f32(reinterpret_cast<float*>(aux), nullptr, 4, st);
}
void use_bwd_aux(const hta::BwdPrep& p, hta::BwdLaunch& b) {
    b.gmax = p.gmax;
    b.q16 = p.q16;
    b.k16 = p.k16;
}

hta::BwdLaunch bwd_base(const hta_shape* s, const void* q, const void* k, const void* v, void* dq,
                        void* dk, void* dv, float scale, const hta::WinTaps& t) {
    hta::BwdLaunch b;
    memset(&b, 0, sizeof(b));
    b.q = q; b.k = k; b.v = v; b.dq = dq; b.dk = dk; b.dv = dv;
    b.out_f32 = s->dtype == HTA_F32 ? 1 : 0;
    b.bh_elems = (long long)s->T * s->P * s->dk;
    b.BH = s->B * s->H;
    b.P = s->P;
    b.T = s->T;
    b.d = s->dk;
    b.dtype = s->dtype;
    b.scale = attn_scale_of(scale, s->dk);
    b.ntaps = t.nA;
    for (int j = 0; j < t.nA; ++j) b.off[j] = t.offA[j];
    return b;
}

// prep (stats, and dout in bf16 if needed) into ws, then the query and key passes.
hipError_t run_window_bwd(const hta_shape* s, hta::BwdLaunch b, const void* o, const float* lse,
                          const void* dout, void* ws, hipStream_t st) {
    char* w = static_cast<char*>(ws);
    hta::BwdPrep p;
    memset(&p, 0, sizeof(p));
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.stats = reinterpret_cast<float*>(w);
    p.rows = (long long)s->B * s->H * s->T * s->P;
    p.d = s->dv;
    p.o_f32 = p.do_f32 = s->out_dtype == HTA_F32 ? 1 : 0;
    p.round_do = s->dtype == HTA_BF16 ? 1 : 0;
    p.q = b.q; p.k = b.k; p.v = b.v;
    char* aux = w + attn_bwd_stats_bytes(s);
    if (do_copy_bytes(s)) p.dout_bf16 = aux + attn_bwd_aux_bytes(s);
    hipError_t e = bind_bwd_aux(s, aux, p, st);
    if (e != hipSuccess) return e;
    if ((e = hta::launch_win_bwd_prep(p, st)) != hipSuccess) return e;
    b.stats = p.stats;
    b.dout = p.dout_bf16 ? p.dout_bf16 : dout;
    use_bwd_aux(p, b);
    return hta::launch_win_bwd(b, st);
}

// Hybrid backward workspace: [GLA backward][stats SWA][stats DSWA][maxima, fp16
// q and k][dout bf16][fp32 partials dq, dk, dv of the GLA branch][the same of
// the SWA branch].
size_t hybrid_bwd_ws(const hta_shape* s) {
    return gla_bwd_ws(s) + 2 * attn_bwd_stats_bytes(s) + attn_bwd_aux_bytes(s) +
           do_copy_bytes(s) + 6 * fp32_seq_bytes(s);
}

}  // namespace

extern "C" {

const char* hta_status_string(int status) {
    switch (status) {
        case HTA_OK: return "HTA_OK";
        case HTA_ERR_NULL: return "HTA_ERR_NULL: a required pointer is NULL";
        case HTA_ERR_SHAPE: return "HTA_ERR_SHAPE: invalid or too large shape";
        case HTA_ERR_WINDOW: return "HTA_ERR_WINDOW: window, taps or dilation out of range";
        case HTA_ERR_DTYPE: return "HTA_ERR_DTYPE: dtype must be HTA_F32 or HTA_BF16";
        case HTA_ERR_UNSUPPORTED: return "HTA_ERR_UNSUPPORTED: head dim, chunk or scale not supported";
        case HTA_ERR_WORKSPACE: return "HTA_ERR_WORKSPACE: workspace missing or too small";
        case HTA_ERR_RING: return "HTA_ERR_RING: ring buffer shorter than the attention windows";
        case HTA_ERR_HIP: return "HTA_ERR_HIP: a HIP runtime call failed";
        case HTA_ERR_ALIAS: return "HTA_ERR_ALIAS: an output overlaps an input";
        case HTA_ERR_ALIGN: return "HTA_ERR_ALIGN: a device pointer is not aligned as required";
        case HTA_ERR_SCRATCH:
            return "HTA_ERR_SCRATCH: the step needs more than the library's fixed scratch "
                   "(HTA_NOALLOC_SCRATCH_BYTES); use hta_stream_step with a workspace";
        default: return "unknown hta status";
    }
}

int hta_last_hip_error(void) { return g_last_hip_error; }

const char* hta_version(void) { return "hta 0.1.0 gfx950"; }

size_t hta_workspace_bytes(int op, const hta_shape* shape, const hta_params* params) {
    if (check_shape(shape) != HTA_OK) return 0;
    if (op == HTA_OP_GLA) {
        if (!params || check_chunk(shape->dtype, params->gla_chunk) != HTA_OK) return 0;
        return gla_ws(shape, params->gla_chunk);
    }
    if (op == HTA_OP_ATTN_BWD) return attn_bwd_ws(shape);
    if (op == HTA_OP_SWA_DSWA) return swa_dswa_ws(shape);
    if (op == HTA_OP_HYBRID_BWD) {
        if (check_params(shape, params) != HTA_OK) return 0;
        return hybrid_bwd_ws(shape);
    }
    if (op == HTA_OP_GLA_BWD) {
        if (!params || check_chunk(shape->dtype, params->gla_chunk) != HTA_OK) return 0;
        return gla_bwd_ws(shape);
    }
    if (op == HTA_OP_HYBRID || op == HTA_OP_STREAM_STEP) {
        if (check_params(shape, params) != HTA_OK) return 0;
        if (op == HTA_OP_STREAM_STEP && shape->T != 1) return 0;
        return gla_ws(shape, params->gla_chunk) + partial_ws(shape);
    }
    return 0;
}

static int window_fwd(int kind, const hta_shape* s, const void* q, const void* k, const void* v,
                      void* o, int a, int b, float scale, void* stream) {
    int st;
    if ((st = check_shape(s)) != HTA_OK) return st;
    if (!q || !k || !v || !o) return HTA_ERR_NULL;
    if ((st = check_align(15, q, k, v, o)) != HTA_OK) return st;
    if ((st = (kind == 0 ? check_window(a) : check_dilated(a, b))) != HTA_OK) return st;
    if ((st = check_scale(scale)) != HTA_OK) return st;
    const size_t nq = seq_bytes(s, s->dk), nv = seq_bytes(s, s->dv);
    const Range ro = range_of(o, out_bytes(s));
    if (overlap(ro, range_of(q, nq)) || overlap(ro, range_of(k, nq)) || overlap(ro, range_of(v, nv)))
        return HTA_ERR_ALIAS;
    hta::WinLaunch w = win_base(s, q, k, v, o, scale);
    w.nbr = 1;
    if (kind == 0) taps_swa(w.taps, a);
    else taps_dswa(w.taps, a, b);
    hipError_t e = hta::launch_win_attn(w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_swa_fwd(const hta_shape* shape, const void* q, const void* k, const void* v, void* o,
                int window_frames, float scale, void* stream) {
    return window_fwd(0, shape, q, k, v, o, window_frames, 0, scale, stream);
}

int hta_dswa_fwd(const hta_shape* shape, const void* q, const void* k, const void* v, void* o,
                 int taps, int dilation_frames, float scale, void* stream) {
    return window_fwd(1, shape, q, k, v, o, taps, dilation_frames, scale, stream);
}

static int window_fwd_lse(int kind, const hta_shape* s, const void* q, const void* k,
                          const void* v, void* o, float* lse, int a, int b, float scale,
                          void* stream) {
    int st;
    if ((st = check_shape(s)) != HTA_OK) return st;
    if (!q || !k || !v || !o || !lse) return HTA_ERR_NULL;
    if ((st = check_align(15, q, k, v, o)) != HTA_OK || (st = check_align(3, lse)) != HTA_OK)
        return st;
    if ((st = (kind == 0 ? check_window(a) : check_dilated(a, b))) != HTA_OK) return st;
    if ((st = check_scale(scale)) != HTA_OK) return st;
    const size_t nq = seq_bytes(s, s->dk), nv = seq_bytes(s, s->dv);
    const Range in[3] = {range_of(q, nq), range_of(k, nq), range_of(v, nv)};
    const Range ro = range_of(o, out_bytes(s)), rl = range_of(lse, gate_bytes(s));
    for (int j = 0; j < 3; ++j)
        if (overlap(ro, in[j]) || overlap(rl, in[j])) return HTA_ERR_ALIAS;
    if (overlap(ro, rl)) return HTA_ERR_ALIAS;
    hta::WinLaunch w = win_base(s, q, k, v, o, scale);
    w.nbr = 1;
    w.lse = lse;
    if (kind == 0) taps_swa(w.taps, a);
    else taps_dswa(w.taps, a, b);
    hipError_t e = hta::launch_win_attn(w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_swa_fwd_lse(const hta_shape* shape, const void* q, const void* k, const void* v, void* o,
                    float* lse, int window_frames, float scale, void* stream) {
    return window_fwd_lse(0, shape, q, k, v, o, lse, window_frames, 0, scale, stream);
}

int hta_dswa_fwd_lse(const hta_shape* shape, const void* q, const void* k, const void* v,
                     void* o, float* lse, int taps, int dilation_frames, float scale,
                     void* stream) {
    return window_fwd_lse(1, shape, q, k, v, o, lse, taps, dilation_frames, scale, stream);
}

static int window_bwd(int kind, const hta_shape* s, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, int a, int b, float scale, void* ws, size_t ws_bytes,
                      void* stream) {
    int st;
    if ((st = check_shape(s)) != HTA_OK) return st;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return HTA_ERR_NULL;
    if ((st = (kind == 0 ? check_window(a) : check_dilated(a, b))) != HTA_OK) return st;
    if ((st = check_scale(scale)) != HTA_OK) return st;
    const size_t need = attn_bwd_ws(s);
    if (!ws || ws_bytes < need) return HTA_ERR_WORKSPACE;
    if ((st = check_align(15, q, k, v, o, dout, dq, dk, dv, ws)) != HTA_OK ||
        (st = check_align(3, lse)) != HTA_OK)
        return st;
    const size_t nq = seq_bytes(s, s->dk), nv = seq_bytes(s, s->dv);
    const Range in[6] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                         range_of(o, out_bytes(s)), range_of(lse, gate_bytes(s)),
                         range_of(dout, out_bytes(s))};
    const Range outs[4] = {range_of(dq, nq), range_of(dk, nq), range_of(dv, nv),
                           range_of(ws, need)};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], in[j])) return HTA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return HTA_ERR_ALIAS;
    }
    hta::WinTaps t;
    if (kind == 0) taps_swa(t, a);
    else taps_dswa(t, a, b);
    hta::BwdLaunch bl = bwd_base(s, q, k, v, dq, dk, dv, scale, t);
    hipError_t e = run_window_bwd(s, bl, o, lse, dout, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_swa_bwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                int window_frames, float scale, void* workspace, size_t workspace_bytes,
                void* stream) {
    return window_bwd(0, shape, q, k, v, o, lse, dout, dq, dk, dv, window_frames, 0, scale,
                      workspace, workspace_bytes, stream);
}

int hta_dswa_bwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 int taps, int dilation_frames, float scale, void* workspace,
                 size_t workspace_bytes, void* stream) {
    return window_bwd(1, shape, q, k, v, o, lse, dout, dq, dk, dv, taps, dilation_frames, scale,
                      workspace, workspace_bytes, stream);
}

int hta_swa_dswa_fwd(const hta_shape* s, const hta_params* p, const void* q, const void* k,
                     const void* v, const float* add, void* o, void* stream) {
    int st;
    if ((st = check_shape(s)) != HTA_OK) return st;
    if (!p) return HTA_ERR_NULL;
    if ((st = check_window(p->swa_window)) != HTA_OK) return st;
    if ((st = check_dilated(p->dswa_taps, p->dswa_dilation)) != HTA_OK) return st;
    if ((st = check_scale(p->attn_scale)) != HTA_OK) return st;
    if (!q || !k || !v || !o) return HTA_ERR_NULL;
    if ((st = check_align(15, q, k, v, o, add)) != HTA_OK) return st;
    const size_t nq = seq_bytes(s, s->dk), nv = seq_bytes(s, s->dv);
    const Range rq = range_of(q, nq), rk = range_of(k, nq), rv = range_of(v, nv);
    const Range ro = range_of(o, out_bytes(s));
    if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv)) return HTA_ERR_ALIAS;
    if (add) {
        const Range ra = range_of(add, (size_t)s->B * s->H * (size_t)s->T * s->P * s->dv * 4);
        if (overlap(ra, rq) || overlap(ra, rk) || overlap(ra, rv)) return HTA_ERR_ALIAS;
        const bool in_place = static_cast<const void*>(add) == o && s->out_dtype == HTA_F32;
        if (!in_place && overlap(ra, ro)) return HTA_ERR_ALIAS;
    }
    hta::WinLaunch w = win_base(s, q, k, v, o, p->attn_scale);
    w.add = add;
    hipError_t e = run_swa_dswa(w, p->swa_window, p->dswa_taps, p->dswa_dilation,
                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_swa_dswa_fwd_ex(const hta_shape* s, const hta_params* p, const void* q, const void* k,
                        const void* v, const float* add, void* o, void* workspace,
                        size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_shape(s)) != HTA_OK) return st;
    if (!p) return HTA_ERR_NULL;
    if ((st = check_window(p->swa_window)) != HTA_OK) return st;
    if ((st = check_dilated(p->dswa_taps, p->dswa_dilation)) != HTA_OK) return st;
    if ((st = check_scale(p->attn_scale)) != HTA_OK) return st;
    if (s->dtype != HTA_BF16)   // fp32 inputs: the two-accumulator pass needs no workspace
        return hta_swa_dswa_fwd(s, p, q, k, v, add, o, stream);
    if (!q || !k || !v || !o) return HTA_ERR_NULL;
    const size_t need = swa_dswa_ws(s);
    if (!workspace || workspace_bytes < need) return HTA_ERR_WORKSPACE;
    if ((st = check_align(15, q, k, v, o, add, workspace)) != HTA_OK) return st;
    const size_t nq = seq_bytes(s, s->dk), nv = seq_bytes(s, s->dv);
    const Range rq = range_of(q, nq), rk = range_of(k, nq), rv = range_of(v, nv);
    const Range ro = range_of(o, out_bytes(s)), rw = range_of(workspace, need);
    if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rw, ro) ||
        overlap(rw, rq) || overlap(rw, rk) || overlap(rw, rv))
        return HTA_ERR_ALIAS;
    if (add) {
        const Range ra = range_of(add, (size_t)s->B * s->H * (size_t)s->T * s->P * s->dv * 4);
        if (overlap(ra, rq) || overlap(ra, rk) || overlap(ra, rv) || overlap(ra, rw)) return HTA_ERR_ALIAS;
        const bool in_place = static_cast<const void*>(add) == o && s->out_dtype == HTA_F32;
        if (!in_place && overlap(ra, ro)) return HTA_ERR_ALIAS;
    }
    char* w = static_cast<char*>(workspace);
    hta::WinLaunch f = win_base(s, q, k, v, o, p->attn_scale);
    f.nbr = 3;
    taps_hybrid(f.taps, p->swa_window, p->dswa_taps, p->dswa_dilation);
    f.park = reinterpret_cast<float*>(w);
    // branch A's output: o itself when o is fp32 and nothing is added in place
    f.oa = (s->out_dtype == HTA_F32 && static_cast<const void*>(add) != o)
               ? static_cast<float*>(o) : reinterpret_cast<float*>(w + park_ws(s));
    f.add = add;
    hipError_t e = hta::launch_win_attn(f, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

static int check_gla_buffers(const hta_shape* s, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* state,
                             const void* o, const void* ws, size_t ws_bytes, size_t ws_need) {
    if (!q || !k || !v || !alpha || !beta || !state || !o) return HTA_ERR_NULL;
    if (!ws || ws_bytes < ws_need) return HTA_ERR_WORKSPACE;
    int st;
    if ((st = check_align(15, q, k, v, o, state, ws)) != HTA_OK ||
        (st = check_align(3, alpha, beta)) != HTA_OK)
        return st;
    const size_t nq = seq_bytes(s, s->dk), nv = seq_bytes(s, s->dv);
    const Range in[5] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                         range_of(alpha, gate_bytes(s)), range_of(beta, gate_bytes(s))};
    const Range outs[3] = {range_of(o, out_bytes(s)), range_of(state, state_bytes(s)),
                           range_of(ws, ws_need)};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlap(outs[i], in[j])) return HTA_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return HTA_ERR_ALIAS;
    }
    return HTA_OK;
}

int hta_gla_fwd(const hta_shape* shape, const void* q, const void* k, const void* v,
                const float* alpha, const float* beta, float* state, void* o, int chunk,
                float scale, void* workspace, size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_shape(shape)) != HTA_OK) return st;
    if ((st = check_chunk(shape->dtype, chunk)) != HTA_OK) return st;
    if (!isfinite(scale)) return HTA_ERR_UNSUPPORTED;
    const size_t need = gla_ws(shape, chunk);
    if ((st = check_gla_buffers(shape, q, k, v, alpha, beta, state, o, workspace, workspace_bytes,
                                need)) != HTA_OK)
        return st;
    hta::GlaLaunch g = gla_base(shape, q, k, v, alpha, beta, state, o, chunk, scale, workspace, need);
    hipError_t e = run_gla(g, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_gla_fwd_ex(const hta_shape* shape, const hta_params* params, const void* q, const void* k,
                   const void* v, const float* alpha, const float* beta, float* state, void* o,
                   void* workspace, size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_shape(shape)) != HTA_OK) return st;
    if (!params) return HTA_ERR_NULL;
    if ((st = check_chunk(shape->dtype, params->gla_chunk)) != HTA_OK) return st;
    if (!isfinite(params->gla_scale)) return HTA_ERR_UNSUPPORTED;
    if (params->gla_form != HTA_GLA_GATED_DELTA && params->gla_form != HTA_GLA_PRINTED)
        return HTA_ERR_UNSUPPORTED;
    const size_t need = gla_ws(shape, params->gla_chunk);
    if ((st = check_gla_buffers(shape, q, k, v, alpha, beta, state, o, workspace, workspace_bytes,
                                need)) != HTA_OK)
        return st;
    hta::GlaLaunch g = gla_base(shape, q, k, v, alpha, beta, state, o, params->gla_chunk,
                                params->gla_scale, workspace, need, params->gla_form);
    hipError_t e = run_gla(g, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_gla_bwd(const hta_shape* shape, const hta_params* params, const void* q, const void* k,
                const void* v, const float* alpha, const float* beta, const float* state0,
                const void* dout, float* dstate, void* dq, void* dk, void* dv, float* dalpha,
                float* dbeta, void* workspace, size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_shape(shape)) != HTA_OK) return st;
    if (!params) return HTA_ERR_NULL;
    if ((st = check_chunk(shape->dtype, params->gla_chunk)) != HTA_OK) return st;
    if (!isfinite(params->gla_scale)) return HTA_ERR_UNSUPPORTED;
    if (params->gla_form != HTA_GLA_GATED_DELTA && params->gla_form != HTA_GLA_PRINTED)
        return HTA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !alpha || !beta || !state0 || !dout || !dstate || !dq || !dk || !dv ||
        !dalpha || !dbeta)
        return HTA_ERR_NULL;
    const size_t need = gla_bwd_ws(shape);
    if (!workspace || workspace_bytes < need) return HTA_ERR_WORKSPACE;
    if ((st = check_align(15, q, k, v, state0, dout, dstate, dq, dk, dv, workspace)) != HTA_OK ||
        (st = check_align(3, alpha, beta, dalpha, dbeta)) != HTA_OK)
        return st;
    const size_t nq = seq_bytes(shape, shape->dk), nv = seq_bytes(shape, shape->dv);
    const Range in[7] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                         range_of(alpha, gate_bytes(shape)), range_of(beta, gate_bytes(shape)),
                         range_of(state0, state_bytes(shape)), range_of(dout, out_bytes(shape))};
    const Range outs[7] = {range_of(dq, nq), range_of(dk, nq), range_of(dv, nv),
                           range_of(dalpha, gate_bytes(shape)), range_of(dbeta, gate_bytes(shape)),
                           range_of(dstate, state_bytes(shape)), range_of(workspace, need)};
    for (int i = 0; i < 7; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlap(outs[i], in[j])) return HTA_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (overlap(outs[i], outs[j])) return HTA_ERR_ALIAS;
    }
    hta::GlaBwdLaunch b = gla_bwd_base(shape, params, q, k, v, alpha, beta, state0, dout, dstate,
                                       dq, dk, dv, dalpha, dbeta, workspace, need);
    hipError_t e = hta::launch_gla_bwd(b, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

size_t hta_hybrid_saved_bytes(const hta_shape* shape) {
    if (check_shape(shape) != HTA_OK) return 0;
    return saved_bytes(shape);
}

int hta_hybrid_fwd_train(const hta_shape* shape, const hta_params* params, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         float* state, void* o, void* saved, void* workspace,
                         size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_shape(shape)) != HTA_OK) return st;
    if ((st = check_params(shape, params)) != HTA_OK) return st;
    if (!saved) return HTA_ERR_NULL;
    const size_t need_gla = gla_ws(shape, params->gla_chunk);
    const size_t need = need_gla + partial_ws(shape);
    if ((st = check_gla_buffers(shape, q, k, v, alpha, beta, state, o, workspace, workspace_bytes,
                                need)) != HTA_OK)
        return st;
    if ((st = check_align(15, saved)) != HTA_OK) return st;
    const size_t nq = seq_bytes(shape, shape->dk), nv = seq_bytes(shape, shape->dv);
    const Range rs = range_of(saved, saved_bytes(shape));
    const Range others[8] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                             range_of(alpha, gate_bytes(shape)), range_of(beta, gate_bytes(shape)),
                             range_of(state, state_bytes(shape)), range_of(o, out_bytes(shape)),
                             range_of(workspace, need)};
    for (int j = 0; j < 8; ++j)
        if (overlap(rs, others[j])) return HTA_ERR_ALIAS;
    hipStream_t sm = static_cast<hipStream_t>(stream);
    const Saved sv = saved_of(shape, saved);
    const long long BH = (long long)shape->B * shape->H;
    hipError_t e = hta::launch_fill_f32(sv.state0, state, BH * shape->dk * shape->dv, sm);
    if (e != hipSuccess) return hip_fail(e);
    hta::WinLaunch w = win_base(shape, q, k, v, o, params->attn_scale);
    if (shape->dtype == HTA_BF16) {
        // the inference forward's GLA branch and one-pass attention, writing what the
        // backward reads besides o: the SWA output and both branches' log-sum-exp
        char* wsb = static_cast<char*>(workspace);
        hta::GlaLaunch g = gla_base(shape, q, k, v, alpha, beta, state, nullptr, params->gla_chunk,
                                    params->gla_scale, workspace, need_gla, params->gla_form);
        TrainOut tr;
        tr.lse_a = sv.lse_swa;
        tr.lse_b = sv.lse_dswa;
        tr.obr_b = sv.o_dswa;
        e = run_hybrid(g, w, partials_of(shape, wsb + need_gla, o), params, sm, tr, sv.o_swa);
        return e == hipSuccess ? HTA_OK : hip_fail(e);
    }
    // fp32: GLA into o, the SWA pass into saved, the DSWA pass adding both into o
    hta::GlaLaunch g = gla_base(shape, q, k, v, alpha, beta, state, o, params->gla_chunk,
                                params->gla_scale, workspace, need_gla, params->gla_form);
    if ((e = run_gla(g, sm)) != hipSuccess) return hip_fail(e);
    hta::WinLaunch a = w;
    a.nbr = 1;
    taps_swa(a.taps, params->swa_window);
    a.o = sv.o_swa;
    a.lse = sv.lse_swa;
    if ((e = hta::launch_win_attn(a, sm)) != hipSuccess) return hip_fail(e);
    hta::WinLaunch d = w;
    d.nbr = 1;
    taps_dswa(d.taps, params->dswa_taps, params->dswa_dilation);
    d.add = static_cast<const float*>(o);
    d.add2 = sv.o_swa;
    d.lse = sv.lse_dswa;
    d.obr = sv.o_dswa;
    e = hta::launch_win_attn(d, sm);
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_hybrid_bwd(const hta_shape* shape, const hta_params* params, const void* q, const void* k,
                   const void* v, const float* alpha, const float* beta, const void* saved,
                   const void* dout, float* dstate, void* dq, void* dk, void* dv, float* dalpha,
                   float* dbeta, void* workspace, size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_shape(shape)) != HTA_OK) return st;
    if ((st = check_params(shape, params)) != HTA_OK) return st;
    if (!q || !k || !v || !alpha || !beta || !saved || !dout || !dstate || !dq || !dk || !dv ||
        !dalpha || !dbeta)
        return HTA_ERR_NULL;
    const size_t need = hybrid_bwd_ws(shape);
    if (!workspace || workspace_bytes < need) return HTA_ERR_WORKSPACE;
    if ((st = check_align(15, q, k, v, saved, dout, dstate, dq, dk, dv, workspace)) != HTA_OK ||
        (st = check_align(3, alpha, beta, dalpha, dbeta)) != HTA_OK)
        return st;
    const size_t nq = seq_bytes(shape, shape->dk), nv = seq_bytes(shape, shape->dv);
    const Range in[7] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                         range_of(alpha, gate_bytes(shape)), range_of(beta, gate_bytes(shape)),
                         range_of(saved, saved_bytes(shape)), range_of(dout, out_bytes(shape))};
    const Range outs[7] = {range_of(dq, nq), range_of(dk, nq), range_of(dv, nv),
                           range_of(dalpha, gate_bytes(shape)), range_of(dbeta, gate_bytes(shape)),
                           range_of(dstate, state_bytes(shape)), range_of(workspace, need)};
    for (int i = 0; i < 7; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlap(outs[i], in[j])) return HTA_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (overlap(outs[i], outs[j])) return HTA_ERR_ALIAS;
    }
    hipStream_t sm = static_cast<hipStream_t>(stream);
    const Saved sv = saved_of(shape, const_cast<void*>(saved));
    char* w = static_cast<char*>(workspace);
    const size_t gws = gla_bwd_ws(shape);
    float* stats_a = reinterpret_cast<float*>(w + gws);
    float* stats_b = reinterpret_cast<float*>(w + gws + attn_bwd_stats_bytes(shape));
    char* aux = w + gws + 2 * attn_bwd_stats_bytes(shape);
    char* p = aux + attn_bwd_aux_bytes(shape);
    void* do_bf16 = nullptr;
    if (do_copy_bytes(shape)) {
        do_bf16 = p;
        p += do_copy_bytes(shape);
    }
    const size_t fs = fp32_seq_bytes(shape);
    float* gq = reinterpret_cast<float*>(p);            // GLA partials
    float* gk = reinterpret_cast<float*>(p + fs);
    float* gv = reinterpret_cast<float*>(p + 2 * fs);
    float* sq = reinterpret_cast<float*>(p + 3 * fs);   // SWA partials
    float* sk = reinterpret_cast<float*>(p + 4 * fs);
    float* sv_ = reinterpret_cast<float*>(p + 5 * fs);
    hta::BwdPrep pr;
    memset(&pr, 0, sizeof(pr));
    pr.dout = dout;
    pr.rows = (long long)shape->B * shape->H * shape->T * shape->P;
    pr.d = shape->dv;
    pr.o_f32 = 1;
    pr.do_f32 = shape->out_dtype == HTA_F32 ? 1 : 0;
    pr.round_do = shape->dtype == HTA_BF16 ? 1 : 0;
    pr.q = q; pr.k = k; pr.v = v;
    hipError_t e;
    if ((e = bind_bwd_aux(shape, aux, pr, sm)) != hipSuccess) return hip_fail(e);
    hta::WinTaps ts, td;
    taps_swa(ts, params->swa_window);
    taps_dswa(td, params->dswa_taps, params->dswa_dilation);
    hta::GlaBwdLaunch gb = gla_bwd_base(shape, params, q, k, v, alpha, beta, sv.state0, dout,
                                        dstate, gq, gk, gv, dalpha, dbeta, w, gws);
    gb.grad_f32 = 1;
    hta::BwdLaunch bs = bwd_base(shape, q, k, v, sq, sk, sv_, params->attn_scale, ts);
    bs.dout = do_bf16 ? do_bf16 : dout;
    bs.stats = stats_a;
    bs.out_f32 = 1;
    hta::BwdLaunch bd = bwd_base(shape, q, k, v, dq, dk, dv, params->attn_scale, td);
    bd.dout = do_bf16 ? do_bf16 : dout;
    bd.stats = stats_b;
    bd.add_q = sq; bd.add_k = sk; bd.add_v = sv_;
    bd.add2_q = gq; bd.add2_k = gk; bd.add2_v = gv;
    use_bwd_aux(pr, bs);
    use_bwd_aux(pr, bd);
    // the first prep (SWA) also makes the fp16 copies and the maxima; the second
    // only its own statistics
    hta::BwdPrep pr2 = pr;
    pr2.q16 = nullptr; pr2.k16 = nullptr; pr2.gmax = nullptr; pr2.dout_bf16 = nullptr;
    pr2.o = sv.o_dswa; pr2.lse = sv.lse_dswa; pr2.stats = stats_b;
    const Side d = side_of(params);
    if (d.s) {
        // The GLA backward (two latency-bound chunk scans with few workgroups, and a
        // chunk-parallel gradient kernel) on `sm`, beside the SWA backward on the
        // caller's side stream; the DSWA backward then adds both sets of partials.
        if ((e = fork(d, sm)) != hipSuccess) return hip_fail(e);
        if ((e = hta::launch_gla_bwd(gb, sm)) != hipSuccess) return hip_fail(e);
        pr.o = sv.o_swa; pr.lse = sv.lse_swa; pr.stats = stats_a; pr.dout_bf16 = do_bf16;
        if ((e = hta::launch_win_bwd_prep(pr, d.s)) != hipSuccess) return hip_fail(e);
        if ((e = hta::launch_win_bwd(bs, d.s)) != hipSuccess) return hip_fail(e);
        if ((e = hta::launch_win_bwd_prep(pr2, sm)) != hipSuccess) return hip_fail(e);
        if ((e = join(d, sm)) != hipSuccess) return hip_fail(e);
        e = hta::launch_win_bwd(bd, sm);
        return e == hipSuccess ? HTA_OK : hip_fail(e);
    }
    if ((e = hta::launch_gla_bwd(gb, sm)) != hipSuccess) return hip_fail(e);
    pr.o = sv.o_swa; pr.lse = sv.lse_swa; pr.stats = stats_a; pr.dout_bf16 = do_bf16;
    if ((e = hta::launch_win_bwd_prep(pr, sm)) != hipSuccess) return hip_fail(e);
    if ((e = hta::launch_win_bwd(bs, sm)) != hipSuccess) return hip_fail(e);
    if ((e = hta::launch_win_bwd_prep(pr2, sm)) != hipSuccess) return hip_fail(e);
    e = hta::launch_win_bwd(bd, sm);
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_hybrid_fwd(const hta_shape* shape, const hta_params* params, const void* q, const void* k,
                   const void* v, const float* alpha, const float* beta, float* state, void* o,
                   void* workspace, size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_shape(shape)) != HTA_OK) return st;
    if ((st = check_params(shape, params)) != HTA_OK) return st;
    const size_t need_gla = gla_ws(shape, params->gla_chunk);
    const size_t need = need_gla + partial_ws(shape);
    if ((st = check_gla_buffers(shape, q, k, v, alpha, beta, state, o, workspace, workspace_bytes,
                                need)) != HTA_OK)
        return st;
    hipStream_t sm = static_cast<hipStream_t>(stream);
    char* wsb = static_cast<char*>(workspace);
    if (shape->dtype == HTA_BF16) {
        hta::GlaLaunch g = gla_base(shape, q, k, v, alpha, beta, state, nullptr, params->gla_chunk,
                                    params->gla_scale, workspace, need_gla, params->gla_form);
        hta::WinLaunch w = win_base(shape, q, k, v, o, params->attn_scale);
        hipError_t e = run_hybrid(g, w, partials_of(shape, wsb + need_gla, o), params, sm);
        return e == hipSuccess ? HTA_OK : hip_fail(e);
    }
    // fp32 inputs: GLA into o, then SWA + DSWA adding it in place.
    hta::GlaLaunch g = gla_base(shape, q, k, v, alpha, beta, state, o, params->gla_chunk,
                                params->gla_scale, workspace, need_gla, params->gla_form);
    g.out_f32 = 1;
    hipError_t e = run_gla(g, sm);
    if (e != hipSuccess) return hip_fail(e);
    hta::WinLaunch w = win_base(shape, q, k, v, o, params->attn_scale);
    w.add = static_cast<float*>(o);
    e = run_swa_dswa(w, params->swa_window, params->dswa_taps, params->dswa_dilation, sm);
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

int hta_project_fwd(const hta_shape* s, int d_model, const void* x, const void* w, void* q,
                    void* k, void* v, float* alpha, float* beta, int flags, void* stream) {
    if (!s) return HTA_ERR_NULL;
    hta_shape s1 = *s;
    s1.out_dtype = s1.dtype;
    int st;
    if ((st = check_shape(&s1)) != HTA_OK) return st;
    if (s->dtype != HTA_BF16 || s->dk != 128 || s->dv != 128) return HTA_ERR_UNSUPPORTED;
    if (s->H % 4 != 0 || 2 * s->H > 128) return HTA_ERR_UNSUPPORTED;
    if (d_model < 64 || d_model % 64 != 0) return HTA_ERR_UNSUPPORTED;
    if (flags & ~(HTA_NORM_Q | HTA_NORM_K)) return HTA_ERR_UNSUPPORTED;
    if (!x || !w || !q || !k || !v || !alpha || !beta) return HTA_ERR_NULL;
    if ((st = check_align(15, x, w, q, k, v)) != HTA_OK || (st = check_align(3, alpha, beta)) != HTA_OK)
        return st;
    const long long L = (long long)s->T * s->P;
    const long long M = (long long)s->B * L;
    const long long N = 3LL * s->H * 128 + 2LL * s->H;
    if ((double)M * d_model >= (double)(1LL << 62)) return HTA_ERR_SHAPE;
    const long long nmt = (M + 127) / 128;
    if (nmt * (3LL * s->H + 1) > 0x7fffffffLL) return HTA_ERR_SHAPE;
    const size_t nseq = seq_bytes(&s1, 128), ngate = gate_bytes(&s1);
    const Range in[2] = {range_of(x, (size_t)M * d_model * 2), range_of(w, (size_t)d_model * N * 2)};
    const Range out[5] = {range_of(q, nseq), range_of(k, nseq), range_of(v, nseq),
                          range_of(alpha, ngate), range_of(beta, ngate)};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 2; ++j)
            if (overlap(out[i], in[j])) return HTA_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlap(out[i], out[j])) return HTA_ERR_ALIAS;
    }
    hta::ProjLaunch p;
    memset(&p, 0, sizeof(p));
    p.x = x; p.w = w; p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
    p.M = M; p.L = L; p.Dm = d_model; p.N = (int)N; p.H = s->H; p.flags = flags; p.nmt = nmt;
    hipError_t e = hta::launch_project(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HTA_OK : hip_fail(e);
}

static int check_ctx(const hta_stream_ctx* c) {
    if (!c) return HTA_ERR_NULL;
    hta_shape s1 = c->s;
    s1.T = 1;
    int st;
    if ((st = check_shape(&s1)) != HTA_OK) return st;
    if ((st = check_params(&s1, &c->p)) != HTA_OK) return st;
    if (!c->ring_k || !c->ring_v || !c->state) return HTA_ERR_NULL;
    if ((st = check_align(15, c->ring_k, c->ring_v, c->state)) != HTA_OK) return st;
    const long long need = (long long)(c->p.dswa_taps - 1) * c->p.dswa_dilation + 1;
    if (c->R < 1 || c->R < c->p.swa_window || c->R < need) return HTA_ERR_RING;
    if (c->n_frames < 0) return HTA_ERR_SHAPE;
    return HTA_OK;
}

static size_t ring_bytes(const hta_stream_ctx* c, int d) {
    return (size_t)c->s.B * c->s.H * (size_t)c->R * c->s.P * d * elem_bytes(c->s.dtype);
}

int hta_stream_init(hta_stream_ctx* ctx, const void* k_prefix, const void* v_prefix, int T_prefix,
                    const float* state_prefix, void* stream) {
    int st;
    if ((st = check_ctx(ctx)) != HTA_OK) return st;
    if (T_prefix < 0) return HTA_ERR_SHAPE;
    if (T_prefix > 0 && (!k_prefix || !v_prefix)) return HTA_ERR_NULL;
    if ((st = check_align(15, k_prefix, v_prefix, state_prefix)) != HTA_OK) return st;
    const hta_shape& s = ctx->s;
    const int BH = s.B * s.H;
    const Range rk = range_of(ctx->ring_k, ring_bytes(ctx, s.dk));
    const Range rv = range_of(ctx->ring_v, ring_bytes(ctx, s.dv));
    const Range rs = range_of(ctx->state, (size_t)BH * s.dk * s.dv * 4);
    if (overlap(rk, rv) || overlap(rk, rs) || overlap(rv, rs)) return HTA_ERR_ALIAS;
    if (T_prefix > 0) {
        const size_t pb = (size_t)BH * T_prefix * (size_t)s.P * s.dk * elem_bytes(s.dtype);
        const Range pk = range_of(k_prefix, pb), pv = range_of(v_prefix, pb);
        if (overlap(pk, rk) || overlap(pk, rv) || overlap(pk, rs) || overlap(pv, rk) ||
            overlap(pv, rv) || overlap(pv, rs))
            return HTA_ERR_ALIAS;
    }
    if (state_prefix) {
        const Range sp = range_of(state_prefix, (size_t)BH * s.dk * s.dv * 4);
        if (overlap(sp, rk) || overlap(sp, rv) || (overlap(sp, rs) && state_prefix != ctx->state))
            return HTA_ERR_ALIAS;
    }
    hipStream_t sm = static_cast<hipStream_t>(stream);
    const long long fe = (long long)s.P * s.dk;  // elements per frame
    const int nfill = T_prefix < ctx->R ? T_prefix : ctx->R;
    for (int i = 0; i < nfill; ++i) {
        const long long f = (long long)T_prefix - nfill + i;
        const long long slot = f % ctx->R;
        hipError_t e = hta::launch_copy_frames(k_prefix, ctx->ring_k, BH, (long long)T_prefix * fe,
                                               (long long)ctx->R * fe, f * fe, slot * fe, fe,
                                               elem_bytes(s.dtype), sm);
        if (e == hipSuccess)
            e = hta::launch_copy_frames(v_prefix, ctx->ring_v, BH, (long long)T_prefix * fe,
                                        (long long)ctx->R * fe, f * fe, slot * fe, fe,
                                        elem_bytes(s.dtype), sm);
        if (e != hipSuccess) return hip_fail(e);
    }
    if (state_prefix != ctx->state) {
        hipError_t e = hta::launch_fill_f32(ctx->state, state_prefix, (long long)BH * s.dk * s.dv, sm);
        if (e != hipSuccess) return hip_fail(e);
    }
    ctx->n_frames = T_prefix;
    return HTA_OK;
}

// The frame's queries against the ring: frame n in slot n mod R.
static hta::WinLaunch ring_launch(const hta_stream_ctx* ctx, const hta_shape& s, const void* q,
                                  void* o, long long n) {
    hta::WinLaunch w = win_base(&s, q, ctx->ring_k, ctx->ring_v, o, ctx->p.attn_scale);
    w.kv_bh = (long long)ctx->R * s.P * s.dk;
    w.frame0 = n;
    w.R = ctx->R;
    return w;
}

}  // extern "C"

namespace {

// Workspace of one stream step (the frame's GLA blocks, then with o the fp32
// partials of the sum); the context must have passed check_ctx.
size_t stream_step_ws(const hta_stream_ctx* ctx, bool with_o, size_t* need_gla) {
    hta_shape s = ctx->s;
    s.T = 1;
    *need_gla = gla_ws(&s, ctx->p.gla_chunk);
    return *need_gla + (with_o ? partial_ws(&s) : 0);
}

}  // namespace

extern "C" {

int hta_stream_step(hta_stream_ctx* ctx, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, void* o, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_ctx(ctx)) != HTA_OK) return st;
    hta_shape s = ctx->s;
    s.T = 1;
    if (!q || !k || !v || !alpha || !beta) return HTA_ERR_NULL;
    size_t need_gla = 0;
    const size_t need = stream_step_ws(ctx, o != nullptr, &need_gla);
    if (!workspace || workspace_bytes < need) return HTA_ERR_WORKSPACE;
    if ((st = check_align(15, q, k, v, o, workspace)) != HTA_OK ||
        (st = check_align(3, alpha, beta)) != HTA_OK)
        return st;
    const int BH = s.B * s.H;
    const size_t nq = seq_bytes(&s, s.dk), nv = seq_bytes(&s, s.dv);
    const Range in[5] = {range_of(q, nq), range_of(k, nq), range_of(v, nv),
                         range_of(alpha, gate_bytes(&s)), range_of(beta, gate_bytes(&s))};
    const Range outs[5] = {range_of(ctx->ring_k, ring_bytes(ctx, s.dk)),
                           range_of(ctx->ring_v, ring_bytes(ctx, s.dv)),
                           range_of(ctx->state, state_bytes(&s)), range_of(workspace, need),
                           o ? range_of(o, out_bytes(&s)) : Range{0, 0}};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlap(outs[i], in[j])) return HTA_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], outs[j])) return HTA_ERR_ALIAS;
    }
    hipStream_t sm = static_cast<hipStream_t>(stream);
    const long long n = ctx->n_frames;
    const long long slot = n % ctx->R;
    const long long fe = (long long)s.P * s.dk;
    hipError_t e = hipSuccess;
    // 1. K/V of the new frame into ring slot n mod R: for bf16 inputs the GLA prep
    //    copies them while it reads the frame (before anything reads the ring).
    const bool fused_copy = s.dtype == HTA_BF16;
    auto ring_into = [&](hta::GlaLaunch& g) {
        if (!fused_copy) return;
        g.ring_k = ctx->ring_k;
        g.ring_v = ctx->ring_v;
        g.ring_bh = (long long)ctx->R * fe;
        g.ring_off = slot * fe;
    };
    if (!fused_copy) {
        e = hta::launch_copy_frames(k, ctx->ring_k, BH, fe, (long long)ctx->R * fe, 0, slot * fe,
                                    fe, elem_bytes(s.dtype), sm);
        if (e == hipSuccess)
            e = hta::launch_copy_frames(v, ctx->ring_v, BH, fe, (long long)ctx->R * fe, 0,
                                        slot * fe, fe, elem_bytes(s.dtype), sm);
        if (e != hipSuccess) return hip_fail(e);
    }
    // 2. GLA over the frame's P tokens from the carried state (chunks start at
    //    the frame), and 3. the frame's queries over the ring plus the GLA
    //    partial -- the two side by side for bf16 inputs.
    char* wsb = static_cast<char*>(workspace);
    if (o && s.dtype == HTA_BF16) {
        hta::GlaLaunch g = gla_base(&s, q, k, v, alpha, beta, ctx->state, nullptr, ctx->p.gla_chunk,
                                    ctx->p.gla_scale, workspace, need_gla, ctx->p.gla_form);
        ring_into(g);
        e = run_hybrid(g, ring_launch(ctx, s, q, o, n), partials_of(&s, wsb + need_gla, o), &ctx->p,
                           sm);
        if (e != hipSuccess) return hip_fail(e);
    } else {
        hta::GlaLaunch g = gla_base(&s, q, k, v, alpha, beta, ctx->state, o, ctx->p.gla_chunk,
                                    ctx->p.gla_scale, workspace, need_gla, ctx->p.gla_form);
        g.out_f32 = 1;
        ring_into(g);
        e = run_gla(g, sm);
        if (e != hipSuccess) return hip_fail(e);
        if (o) {
            hta::WinLaunch w = ring_launch(ctx, s, q, o, n);
            w.add = static_cast<float*>(o);
            e = run_swa_dswa(w, ctx->p.swa_window, ctx->p.dswa_taps, ctx->p.dswa_dilation, sm);
            if (e != hipSuccess) return hip_fail(e);
        }
    }
    ctx->n_frames = n + 1;
    return HTA_OK;
}

}  // extern "C"

// Scratch of hta_stream_step_noalloc: a fixed array in the library's code
// object, one copy per GPU (allocated when the code object loads on that GPU,
// held until the process ends). In host code `scratch` only stands in for the
// symbol; its device address on each GPU comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[HTA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each GPU (set once)

// The scratch address on `dev`, which must be the current device. The first
// call on a device looks the symbol up; the address never changes after.
int scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return HTA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!ptr) return hip_fail(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return HTA_OK;
}

}  // namespace

extern "C" {

int hta_stream_step_noalloc(hta_stream_ctx* ctx, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, void* o, void* stream) {
    int st;
    if ((st = check_ctx(ctx)) != HTA_OK) return st;
    size_t need_gla = 0;
    if (stream_step_ws(ctx, o != nullptr, &need_gla) > (size_t)HTA_NOALLOC_SCRATCH_BYTES)
        return HTA_ERR_SCRATCH;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (stream) {   // the scratch used must be the copy on the stream's GPU
        hipDevice_t sdev = 0;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) return hip_fail(e);
        if (sdev != dev) return HTA_ERR_UNSUPPORTED;
    }
    void* ws = nullptr;
    if ((st = scratch_on(dev, &ws)) != HTA_OK) return st;
    // Every scratch byte this step reads it has written first in the same call,
    // so nothing needs clearing between calls.
    return hta_stream_step(ctx, q, k, v, alpha, beta, o, ws, (size_t)HTA_NOALLOC_SCRATCH_BYTES,
                           stream);
}

}  // extern "C"
