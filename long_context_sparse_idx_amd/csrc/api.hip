// C-ABI entry points of liblcsi (declared in include/lcsi.h): argument
// validation, workspace sizing and kernel launches.  Every check runs on the
// host before the first launch, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"
#include "lcsi.h"

// Device scratch of sparse_attn_noalloc: the partial results of a decode
// call, held in a file-scope array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in):
// the device address of each GPU's copy comes from hipGetSymbolAddress,
// taken once per device with that device current (scratch_address below),
// and only that address reaches the kernels.
static __device__ __align__(256) uint8_t scratch[LCSI_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace lcsi;

constexpr size_t WS_ALIGN = 256;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool mult(int64_t v, int64_t m) { return v >= 0 && v % m == 0; }

int64_t score_ld(int64_t T_kv) { return (T_kv + 63) / 64 * 64; }

int check_rows(int32_t B, int32_t T_q, int32_t T_kv, int64_t q_pos0, int32_t top_k)
{
    if (B < 1 || T_q < 1 || T_kv < 1 || q_pos0 < 0 || q_pos0 + T_q > (int64_t)T_kv) return LCSI_EINVAL;
    if (top_k < 1) return LCSI_EINVAL;
    if (top_k > LCSI_MAX_TOPK) return LCSI_EUNSUPPORTED;
    return LCSI_OK;
}

int check_indexer(const lcsi_indexer *a, bool preset)
{
    if (!a) return LCSI_EINVAL;
    int rc = check_rows(a->B, a->T_q, a->T_kv, a->q_pos0, a->top_k);
    if (rc || preset) return rc;
    if (a->key_dtype != LCSI_KEY_BF16 && a->key_dtype != LCSI_KEY_FP8_E4M3) return LCSI_EINVAL;
    if (a->q_dtype != LCSI_Q_BF16 && a->q_dtype != LCSI_Q_FP8_E4M3) return LCSI_EINVAL;
    const bool fp8 = a->key_dtype == LCSI_KEY_FP8_E4M3;
    const bool q8 = a->q_dtype == LCSI_Q_FP8_E4M3;
    if (!a->q || !a->k || !a->w || (fp8 && !a->k_scale) || (q8 && !a->q_scale)) return LCSI_EINVAL;
    if (a->H_I < 1 || a->D_I < 1) return LCSI_EINVAL;
    if (a->q_sb < 0 || a->q_st < 0 || a->q_sh < 0 || a->k_sb < 0 || a->k_st < 0 || a->w_sb < 0 || a->w_st < 0 ||
        (fp8 && a->ks_sb < 0) || (q8 && (a->qs_sb < 0 || a->qs_st < 0)))
        return LCSI_EINVAL;
    if (q8 && !fp8) return LCSI_EUNSUPPORTED;  // fp8 x fp8 products need fp8 keys
    const int H = a->H_I;
    if (!(H == 4 || H == 8 || H == 16 || H == 32 || H == 64)) return LCSI_EUNSUPPORTED;
    if (!(a->D_I == 64 || a->D_I == 128)) return LCSI_EUNSUPPORTED;
    // the score rows of one workgroup (512/H rows) are addressed with 32-bit offsets
    if ((int64_t)(512 / H) * score_ld(a->T_kv) * 4 >= ((int64_t)1 << 31)) return LCSI_EUNSUPPORTED;
    // a 128-key tile of keys is addressed with 32-bit offsets
    if (a->k_st * (fp8 ? 1 : 2) * 128 >= ((int64_t)1 << 31)) return LCSI_EUNSUPPORTED;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->w, 16)) return LCSI_EALIGN;
    const int64_t qel = q8 ? 16 : 8;  // query elements per 16 bytes
    if (!mult(a->q_sb, qel) || !mult(a->q_st, qel) || !mult(a->q_sh, qel)) return LCSI_EALIGN;
    if (q8 && !aligned(a->q_scale, 4)) return LCSI_EALIGN;
    const int64_t kel = fp8 ? 16 : 8;  // elements per 16 bytes
    if (!mult(a->k_sb, kel) || !mult(a->k_st, kel)) return LCSI_EALIGN;
    if (!mult(a->w_sb, 4) || !mult(a->w_st, 4)) return LCSI_EALIGN;
    if (fp8 && !aligned(a->k_scale, 4)) return LCSI_EALIGN;
    return LCSI_OK;
}

int check_attn(const lcsi_attn *a)
{
    if (!a) return LCSI_EINVAL;
    int rc = check_rows(a->B, a->T_q, a->T_kv, a->q_pos0, a->top_k);
    if (rc) return rc;
    if (!a->q || !a->k || !a->v || !a->out) return LCSI_EINVAL;
    if (a->H_q < 1 || a->D_qk < 1 || a->D_v < 1 || !isfinite(a->sm_scale) || !(a->sm_scale > 0.f)) return LCSI_EINVAL;
    if (a->q_sb < 0 || a->q_st < 0 || a->q_sh < 0 || a->k_sb < 0 || a->k_st < 0 || a->v_sb < 0 || a->v_st < 0 ||
        a->o_sb < 0 || a->o_st < 0 || a->o_sh < 0)
        return LCSI_EINVAL;
    if (a->H_q > 64) return LCSI_EUNSUPPORTED;
    // KV rows are addressed with 32-bit byte strides
    if (a->k_st * 2 >= ((int64_t)1 << 32) || a->v_st * 2 >= ((int64_t)1 << 32)) return LCSI_EUNSUPPORTED;
    if (!((a->D_qk == 128 && a->D_v == 128) || (a->D_qk == 576 && a->D_v == 512))) return LCSI_EUNSUPPORTED;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->out, 16)) return LCSI_EALIGN;
    if (!mult(a->q_sb, 8) || !mult(a->q_st, 8) || !mult(a->q_sh, 8) || !mult(a->k_sb, 8) || !mult(a->k_st, 8) ||
        !mult(a->v_sb, 8) || !mult(a->v_st, 8) || !mult(a->o_sb, 8) || !mult(a->o_st, 8) || !mult(a->o_sh, 8))
        return LCSI_EALIGN;
    return LCSI_OK;
}

size_t score_rows_bytes(const lcsi_indexer *a)
{
    const size_t s = (size_t)a->B * (size_t)a->T_q * (size_t)score_ld(a->T_kv) * sizeof(float);
    return (s + 255) / 256 * 256;
}

size_t align_ws(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

// Whether a call takes the fused candidate pass (see lcsi.h: LCSI_UNFUSED).
bool fused_plan(const lcsi_indexer *a, unsigned flags)
{
    if (flags & (LCSI_SCORES_PRESET | LCSI_SCORES_ONLY | LCSI_UNFUSED)) return false;
    ScoreArgs sa{};
    sa.B = a->B;
    sa.T_q = a->T_q;
    sa.H = a->H_I;
    sa.q_pos0 = a->q_pos0;
    sa.top_k = a->top_k;
    return score_can_fuse(sa);
}

// score rows, then the selection's own part (few long rows only), then the
// fused pass's counts and candidate slots
size_t score_ws_bytes(const lcsi_indexer *a, unsigned flags)
{
    size_t s = score_rows_bytes(a) + select_ws_bytes(a->B, a->T_q, a->q_pos0);
    if (fused_plan(a, flags)) {
        const size_t rows = (size_t)a->B * (size_t)a->T_q;
        s += align_ws(rows * 4) + align_ws((1 + FUSE_RMAX) * 4) + rows * FUSE_CAP * 8;
    }
    return s;
}

size_t attn_ws_bytes(const lcsi_attn *a, AttnPlan *plan_out = nullptr)
{
    const AttnPlan pl = attn_plan(a->B, a->T_q, a->H_q, a->D_qk, a->top_k);
    if (plan_out) *plan_out = pl;
    if (pl.splits == 1) return 0;
    const size_t rows = (size_t)a->B * a->T_q * pl.splits * a->H_q;
    const size_t o = (rows * a->D_v * sizeof(uint16_t) + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN;  // fp16 O / l
    return o + rows * 2 * sizeof(float);                                                       // fp32 (m, l)
}

// The workspace rule shared by all calls (see lcsi.h).  Returns 1 for query
// mode (requirement stored, nothing to launch), 0 to proceed, <0 on error.
int workspace_rule(const void *ws, size_t *ws_bytes, size_t need)
{
    if (!ws) {
        if (ws_bytes) {
            *ws_bytes = need;
            return 1;
        }
        return need ? LCSI_EWORKSPACE : 0;
    }
    if (!ws_bytes) return LCSI_EINVAL;
    if (*ws_bytes < need) return LCSI_EWORKSPACE;
    if (!aligned(ws, WS_ALIGN)) return LCSI_EALIGN;
    return 0;
}

int check_idx_out(const int32_t *idx, int64_t sb, int64_t st)
{
    if (!idx) return LCSI_EINVAL;
    if (sb < 0 || st < 0) return LCSI_EINVAL;
    if (!aligned(idx, 4)) return LCSI_EALIGN;
    return LCSI_OK;
}

int record(void *const *events, int i, hipStream_t s)
{
    if (!events || !events[i]) return LCSI_OK;
    return hipEventRecord((hipEvent_t)events[i], s) == hipSuccess ? LCSI_OK : LCSI_EHIP;
}

// Launch the indexer steps of one validated call.  ev (optional) points at
// two events recorded after scoring and after selection.
int run_indexer(const lcsi_indexer *a, int32_t *idx, int64_t idx_sb, int64_t idx_st, float *ws, unsigned flags,
                hipStream_t s, void *const *ev)
{
    const int64_t ld = score_ld(a->T_kv);
    const bool fused = fused_plan(a, flags);
    const uint32_t *cand = nullptr;
    const int32_t *ccnt = nullptr;
    if (!(flags & LCSI_SCORES_PRESET)) {
        ScoreArgs sa{};
        sa.B = a->B;
        sa.T_q = a->T_q;
        sa.T_kv = a->T_kv;
        sa.H = a->H_I;
        sa.D = a->D_I;
        sa.fp8 = a->key_dtype == LCSI_KEY_FP8_E4M3;
        sa.q8 = a->q_dtype == LCSI_Q_FP8_E4M3;
        sa.q_pos0 = a->q_pos0;
        const int64_t qbytes = sa.q8 ? 1 : 2;
        sa.q = (const uint8_t *)a->q;
        sa.q_sb = a->q_sb * qbytes;
        sa.q_st = a->q_st * qbytes;
        sa.q_sh = a->q_sh * qbytes;
        sa.q_scale = a->q_scale;
        sa.qs_sb = a->qs_sb;
        sa.qs_st = a->qs_st;
        const int64_t kbytes = sa.fp8 ? 1 : 2;
        sa.k = (const uint8_t *)a->k;
        sa.k_sb = a->k_sb * kbytes;
        sa.k_st = a->k_st * kbytes;
        sa.k_scale = a->k_scale;
        sa.ks_sb = a->ks_sb;
        sa.w = a->w;
        sa.w_sb = a->w_sb;
        sa.w_st = a->w_st;
        sa.S = ws;
        sa.ld = ld;
        sa.key_split = score_key_split(sa);
        sa.top_k = a->top_k;
        if (fused) {
            // workspace past the rows: counts, the list of unsettled rows
            // (its length first), candidate slots
            uint8_t *fz = (uint8_t *)ws + score_rows_bytes(a) + select_ws_bytes(a->B, a->T_q, a->q_pos0);
            sa.ccnt = (int32_t *)fz;
            fz += align_ws((size_t)a->B * a->T_q * 4);
            sa.rcount = (int32_t *)fz;
            sa.rlist = sa.rcount + 1;
            sa.rmax = FUSE_RMAX;
            sa.cand = (uint32_t *)(fz + align_ws((1 + FUSE_RMAX) * 4));
            if (launch_zero_i32(sa.rcount, s) != hipSuccess) return LCSI_EHIP;
            sa.fuse = 1;
            if (launch_score(sa, s) != hipSuccess) return LCSI_EHIP;
            // full rows for the rows the candidates cannot settle (usually
            // none: then every workgroup exits at once): listed rows by the
            // split-key kernel, 64 key ranges each ...
            sa.fuse = 0;
            const int64_t n_keys = a->q_pos0 + a->T_q;
            int64_t ks = (n_keys + 63) / 64;
            ks = (ks + 255) / 256 * 256;
            sa.key_split = score_key_range(ks < 512 ? 512 : ks, sa.k_st);
            if (launch_score(sa, s) != hipSuccess) return LCSI_EHIP;
            // ... and, if the list overflowed, the workgroups holding such rows
            sa.rlist = nullptr;
            sa.redo = sa.ccnt;
            if (launch_score(sa, s) != hipSuccess) return LCSI_EHIP;
            cand = sa.cand;
            ccnt = sa.ccnt;
        } else if (launch_score(sa, s) != hipSuccess) {
            return LCSI_EHIP;
        }
    }
    if (ev && record(ev, 0, s)) return LCSI_EHIP;
    if (!(flags & LCSI_SCORES_ONLY)) {
        SelectArgs se{};
        se.B = a->B;
        se.T_q = a->T_q;
        se.top_k = a->top_k;
        se.q_pos0 = a->q_pos0;
        se.T_kv = a->T_kv;
        se.S = ws;
        se.ld = ld;
        se.idx = idx;
        se.idx_sb = idx_sb;
        se.idx_st = idx_st;
        se.cand = cand;
        se.ccnt = ccnt;
        if (launch_select(se, (uint8_t *)ws + score_rows_bytes(a), s) != hipSuccess) return LCSI_EHIP;
    }
    if (ev && record(ev, 1, s)) return LCSI_EHIP;
    return LCSI_OK;
}

// `host`: an earlier split call's merge for this launch to do first (or
// null); `defer`: if not null, a split call leaves its own merge to the
// caller (in *defer) instead of launching it.
int run_attn(const lcsi_attn *a, const int32_t *idx, int64_t idx_sb, int64_t idx_st, float *ws, hipStream_t s,
             const MergeArgs *host = nullptr, MergeArgs *defer = nullptr)
{
    AttnArgs aa{};
    aa.B = a->B;
    aa.T_q = a->T_q;
    aa.T_kv = a->T_kv;
    aa.H = a->H_q;
    aa.DQK = a->D_qk;
    aa.DV = a->D_v;
    aa.top_k = a->top_k;
    aa.sm_scale_log2 = a->sm_scale * 1.4426950408889634f;
    aa.q_pos0 = a->q_pos0;
    aa.q = (const uint16_t *)a->q;
    aa.q_sb = a->q_sb;
    aa.q_st = a->q_st;
    aa.q_sh = a->q_sh;
    aa.k = (const uint16_t *)a->k;
    aa.k_sb = a->k_sb;
    aa.k_st = a->k_st;
    aa.v = (const uint16_t *)a->v;
    aa.v_sb = a->v_sb;
    aa.v_st = a->v_st;
    aa.out = (uint16_t *)a->out;
    aa.o_sb = a->o_sb;
    aa.o_st = a->o_st;
    aa.o_sh = a->o_sh;
    aa.idx = idx;
    aa.idx_sb = idx_sb;
    aa.idx_st = idx_st;
    AttnPlan pl;
    attn_ws_bytes(a, &pl);
    aa.splits = pl.splits;
    aa.split_len = pl.split_len;
    if (aa.splits > 1) {
        const size_t rows = (size_t)a->B * a->T_q * aa.splits * a->H_q;
        const size_t o = (rows * a->D_v * sizeof(uint16_t) + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN;
        aa.part_o = (uint16_t *)ws;
        aa.part_ml = (float *)((char *)ws + o);
    }
    if (host) aa.mg = *host;
    return launch_attn(aa, s, defer) == hipSuccess ? LCSI_OK : LCSI_EHIP;
}

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_dev[MAX_DEVICES];  // device address of `scratch` per device, guarded by scratch_mu

// The address of the current device's scratch, looked up on the first call
// for that device.  The stream (NULL: the current device's null stream) must
// belong to the current device.
int scratch_address(hipStream_t s, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return LCSI_EHIP;
    if (s) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return LCSI_EHIP;
        if ((int)sdev != dev) return LCSI_EINVAL;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LCSI_EHIP;
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return LCSI_OK;
}

}  // namespace

extern "C" {

int64_t lcsi_score_ld(int32_t T_kv) { return score_ld(T_kv < 0 ? 0 : T_kv); }

int idx_score_topk(const lcsi_indexer *a, int32_t *idx, int64_t idx_sb, int64_t idx_st, float *score_ws,
                   size_t *ws_bytes, unsigned flags, void *stream)
{
    if (flags & ~(LCSI_SCORES_PRESET | LCSI_SCORES_ONLY | LCSI_UNFUSED)) return LCSI_EINVAL;
    if ((flags & LCSI_SCORES_PRESET) && (flags & LCSI_SCORES_ONLY)) return LCSI_EINVAL;
    int rc = check_indexer(a, flags & LCSI_SCORES_PRESET);
    if (rc) return rc;
    if (!score_ws && ws_bytes)
        return workspace_rule(score_ws, ws_bytes, score_ws_bytes(a, flags)) < 0 ? LCSI_EINVAL : LCSI_OK;
    if (!(flags & LCSI_SCORES_ONLY) && (rc = check_idx_out(idx, idx_sb, idx_st))) return rc;
    rc = workspace_rule(score_ws, ws_bytes, score_ws_bytes(a, flags));
    if (rc) return rc < 0 ? rc : LCSI_OK;
    return run_indexer(a, idx, idx_sb, idx_st, score_ws, flags, (hipStream_t)stream, nullptr);
}

int sparse_attn(const lcsi_attn *a, const int32_t *idx, int64_t idx_sb, int64_t idx_st, float *ws,
                size_t *ws_bytes, void *stream)
{
    int rc = check_attn(a);
    if (rc) return rc;
    if (!ws && ws_bytes) return workspace_rule(ws, ws_bytes, attn_ws_bytes(a)) < 0 ? LCSI_EINVAL : LCSI_OK;
    if ((rc = check_idx_out(idx, idx_sb, idx_st))) return rc;
    rc = workspace_rule(ws, ws_bytes, attn_ws_bytes(a));
    if (rc) return rc < 0 ? rc : LCSI_OK;
    return run_attn(a, idx, idx_sb, idx_st, ws, (hipStream_t)stream);
}

int sparse_attn_noalloc(const lcsi_attn *a, const int32_t *idx, int64_t idx_sb, int64_t idx_st, void *stream)
{
    int rc = check_attn(a);
    if (rc) return rc;
    if ((rc = check_idx_out(idx, idx_sb, idx_st))) return rc;
    const size_t need = attn_ws_bytes(a);
    if (need > (size_t)LCSI_NOALLOC_SCRATCH_BYTES) return LCSI_ESCRATCH;
    void *ws = nullptr;
    if (need && (rc = scratch_address((hipStream_t)stream, &ws))) return rc;
    return run_attn(a, idx, idx_sb, idx_st, (float *)ws, (hipStream_t)stream);
}

int run_layer_group(int L, const uint8_t *pattern, const lcsi_indexer *idx_args, int n_idx_args,
                    const lcsi_attn *attn_args, int32_t *idx_cache, int n_slots, int64_t slot_stride,
                    int64_t idx_sb, int64_t idx_st, float *ws, size_t *ws_bytes, void *const *events,
                    void *stream)
{
    if (L < 1 || !pattern || !attn_args || n_slots < 1 || slot_stride < 0) return LCSI_EINVAL;
    int nf = 0;
    for (int l = 0; l < L; ++l) nf += pattern[l] ? 1 : 0;
    if (!pattern[0] || nf != n_idx_args) return LCSI_EPATTERN;
    if (!idx_args) return LCSI_EINVAL;
    int rc;
    size_t need = 0, need_attn = 0;
    const lcsi_attn *a0 = &attn_args[0];
    for (int f = 0; f < nf; ++f) {
        const lcsi_indexer *x = &idx_args[f];
        if ((rc = check_indexer(x, false))) return rc;
        if (x->B != a0->B || x->T_q != a0->T_q || x->q_pos0 != a0->q_pos0 || x->top_k != a0->top_k) return LCSI_EINVAL;
        const size_t s = score_ws_bytes(x, 0u);
        need = s > need ? s : need;
    }
    for (int l = 0; l < L; ++l) {
        const lcsi_attn *y = &attn_args[l];
        if ((rc = check_attn(y))) return rc;
        if (y->B != a0->B || y->T_q != a0->T_q || y->q_pos0 != a0->q_pos0 || y->top_k != a0->top_k) return LCSI_EINVAL;
        const size_t s = attn_ws_bytes(y);
        need_attn = s > need_attn ? s : need_attn;
    }
    // Split (decode) attention: a layer's partial results are merged by the
    // next layer's attention launch (the last layer's by a merge launch of
    // its own), so two partial regions alternate after the indexer's region.
    // (All layers share B, T_q and top_k, so all split or none do.)
    AttnPlan pl0;
    attn_ws_bytes(a0, &pl0);
    const bool defer = pl0.splits > 1;
    const size_t attn_off = defer ? align_ws(need) : 0, attn_reg = align_ws(need_attn);
    need = defer ? attn_off + 2 * attn_reg : (need > need_attn ? need : need_attn);
    if (!ws && ws_bytes) return workspace_rule(ws, ws_bytes, need) < 0 ? LCSI_EINVAL : LCSI_OK;
    if ((rc = check_idx_out(idx_cache, idx_sb, idx_st))) return rc;
    rc = workspace_rule(ws, ws_bytes, need);
    if (rc) return rc < 0 ? rc : LCSI_OK;

    hipStream_t s = (hipStream_t)stream;
    int f = 0;
    int32_t *cur = nullptr;
    MergeArgs pending{};  // the previous layer's merge, still to do (S == 0: none)
    for (int l = 0; l < L; ++l) {
        if ((rc = record(events, 4 * l, s))) return rc;
        if (pattern[l]) {
            cur = idx_cache + (int64_t)(f % n_slots) * slot_stride;
            if ((rc = run_indexer(&idx_args[f], cur, idx_sb, idx_st, ws, 0u, s, events ? events + 4 * l + 1 : nullptr)))
                return rc;
            ++f;
        } else {
            if ((rc = record(events, 4 * l + 1, s)) || (rc = record(events, 4 * l + 2, s))) return rc;
        }
        if (defer) {
            float *pws = (float *)((char *)ws + attn_off + (size_t)(l & 1) * attn_reg);
            MergeArgs own{};
            if ((rc = run_attn(&attn_args[l], cur, idx_sb, idx_st, pws, s, pending.S ? &pending : nullptr, &own)))
                return rc;
            pending = own;
            if (l == L - 1 && pending.S && launch_merge(pending, s) != hipSuccess) return LCSI_EHIP;
        } else if ((rc = run_attn(&attn_args[l], cur, idx_sb, idx_st, ws, s))) {
            return rc;
        }
        if ((rc = record(events, 4 * l + 3, s))) return rc;
    }
    return LCSI_OK;
}

int idx_overlap(const int32_t *a, int64_t a_sb, int64_t a_st, const int32_t *b, int64_t b_sb, int64_t b_st,
                int32_t B, int32_t T_q, int32_t top_k, int32_t *counts, void *stream)
{
    if (B < 1 || T_q < 1 || top_k < 1 || !counts) return LCSI_EINVAL;
    if (top_k > LCSI_MAX_TOPK) return LCSI_EUNSUPPORTED;
    int rc;
    if ((rc = check_idx_out(a, a_sb, a_st)) || (rc = check_idx_out(b, b_sb, b_st))) return rc;
    if (!aligned(counts, 4)) return LCSI_EALIGN;
    OverlapArgs oa{};
    oa.B = B;
    oa.T_q = T_q;
    oa.top_k = top_k;
    oa.a = a;
    oa.a_sb = a_sb;
    oa.a_st = a_st;
    oa.b = b;
    oa.b_sb = b_sb;
    oa.b_st = b_st;
    oa.counts = counts;
    return launch_overlap(oa, (hipStream_t)stream) == hipSuccess ? LCSI_OK : LCSI_EHIP;
}

const char *lcsi_strerror(int code)
{
    switch (code) {
    case LCSI_OK: return "ok";
    case LCSI_EINVAL: return "invalid argument";
    case LCSI_EUNSUPPORTED: return "shape outside the supported kernel envelope";
    case LCSI_EWORKSPACE: return "workspace missing or too small";
    case LCSI_EPATTERN: return "invalid F/S layer pattern";
    case LCSI_EALIGN: return "misaligned pointer or stride";
    case LCSI_EHIP: return "HIP launch error";
    case LCSI_ESCRATCH: return "call needs more than the library's static scratch (sparse_attn_noalloc)";
    default: return "unknown status";
    }
}

}  // extern "C"
