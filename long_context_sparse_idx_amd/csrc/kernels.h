// Internal launch interface between the C-ABI host code (api.hip) and the
// kernels.  Not installed; the public interface is include/lcsi.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcsi {

struct ScoreArgs {
    int B, T_q, T_kv, H, D;
    int fp8;                  // keys fp8 e4m3 (+ per-key scale)
    int q8;                   // queries fp8 e4m3 (+ per-(token, head) scale); needs fp8 keys
    int64_t q_pos0;
    const uint8_t *q;         // bf16 or fp8 rows, strides in BYTES
    int64_t q_sb, q_st, q_sh;
    const float *q_scale;     // fp8 queries only
    int64_t qs_sb, qs_st;
    const uint8_t *k;         // bf16 or fp8 rows, strides in BYTES
    int64_t k_sb, k_st;
    const float *k_scale;     // fp8 only
    int64_t ks_sb;
    const float *w;
    int64_t w_sb, w_st;
    float *S;                 // [B][T_q][ld]
    int64_t ld;
    int key_split;            // keys per workgroup (split-key kernel)
    int top_k;
    // fused selection (prefill kernel, H >= 16): instead of S, each row's
    // scores at or above a sampled threshold go to cand as ascending
    // (score bits, position) pairs, at most FUSE_CAP per row, and ccnt gets
    // the row's count (FUSE_CAP + 1 and above: overflow)
    int fuse;
    uint32_t *cand;           // [B * T_q][FUSE_CAP][2]
    int32_t *ccnt;            // [B * T_q]
    // rescoring after a fused pass (unfused prefill kernel): when set, a
    // workgroup runs only if one of its rows has a count the selection
    // cannot use (fused_row_bad), and then writes its full rows to S
    const int32_t *redo;      // [B * T_q] counts of the fused pass, or null
    // rows the fused pass could not settle: it appends their ids (b*T_q + t)
    // to rlist (the first rmax of them; *rcount counts them all, and must be
    // zero before the pass).  The split-key kernel with rlist set rescores
    // listed rows (blockIdx.y = list entry); the prefill kernel with redo set
    // runs only when the list overflowed.
    int32_t *rlist;           // [rmax]
    int32_t *rcount;
    int rmax;
};

// Candidate slots per row of the fused selection.
constexpr int FUSE_CAP = 16384;

// A fused row of n scores whose count c the selection cannot use: fewer
// candidates than the top-k (the sampled threshold was too high) or more
// than the slots hold.  Rows with n <= k need no selection at all.
__host__ __device__ inline bool fused_row_bad(int32_t c, int64_t n, int k)
{
    return n > k && (c < k || c > FUSE_CAP);
}

struct SelectArgs {
    int B, T_q, top_k;
    int64_t q_pos0, T_kv;
    const float *S;           // [B][T_q][ld]
    int64_t ld;
    int32_t *idx;
    int64_t idx_sb, idx_st;
    // few long rows (set by launch_select from the workspace past the scores)
    int nseg;                 // segments per row
    int64_t seg_len;          // scores per segment
    int32_t *cnt;             // [rows][nseg] candidates per segment (-1: overflow)
    uint32_t *ckey;           // [rows][nseg][cap] candidate keys
    int32_t *cidx;            // [rows][nseg][cap] candidate positions
    // after a fused score pass: the candidate pairs and counts (ScoreArgs);
    // rows with a usable count select from them, the others from S
    const uint32_t *cand;
    const int32_t *ccnt;
};

// The log-sum-exp merge of one split attention call's partial results
// (part_o, part_ml as AttnArgs lays them out) into its bf16 output.
struct MergeArgs {
    const uint16_t *part_o;
    const float *part_ml;
    uint16_t *out;
    int64_t o_sb, o_st, o_sh;
    int rows, T_q, H, DV, S;  // rows = B * T_q; S = splits (0: nothing to merge)
};

struct AttnArgs {
    int B, T_q, T_kv, H, DQK, DV, top_k;
    float sm_scale_log2;      // sm_scale * log2(e)
    int64_t q_pos0;
    const uint16_t *q;
    int64_t q_sb, q_st, q_sh;
    const uint16_t *k;
    int64_t k_sb, k_st;
    const uint16_t *v;
    int64_t v_sb, v_st;
    uint16_t *out;
    int64_t o_sb, o_st, o_sh;
    const int32_t *idx;
    int64_t idx_sb, idx_st;
    int splits;               // key splits per query row (1 = write bf16 directly)
    int split_len;            // index entries per split (multiple of 32)
    int hgroups;              // workgroups sharing one row's heads (each takes H / hgroups of them)
    uint16_t *part_o;         // [B*T_q][splits][H][DV] fp16, the part's O / l (splits > 1)
    float *part_ml;           // [B*T_q][splits][H][2]
    MergeArgs mg;             // another (earlier) split call's merge, done by this launch's workgroups
                              // before their own work (mg.S == 0: none)
};

// How sparse_attn splits each row's index list.  The split count (and so the
// arithmetic of every row) depends only on top_k and on whether the call is a
// decode call (T_q == 1), never on B or on the other rows of the call.
// launch_attn may also share a row's heads out between workgroups, which
// changes no arithmetic.
struct AttnPlan {
    int splits, split_len;
};
AttnPlan attn_plan(int B, int T_q, int H, int DQK, int top_k);

bool score_use_split(const ScoreArgs &a);
// Whether a call with these arguments can take the fused selection.
bool score_can_fuse(const ScoreArgs &a);
int score_key_split(const ScoreArgs &a);
// ks keys per split-key workgroup, lowered to what 32-bit byte offsets reach
// at a key stride of k_st_bytes.
int score_key_range(int64_t ks, int64_t k_st_bytes);
hipError_t launch_score(const ScoreArgs &a, hipStream_t st);
// Zero one int32 in device memory (a kernel, so the call may be captured
// in a graph).
hipError_t launch_zero_i32(int32_t *p, hipStream_t st);
// Rows a rescoring launch takes from the fused pass's list.
constexpr int FUSE_RMAX = 64;
// Workspace bytes the selection needs past the score rows (0 unless few
// long rows take the multi-workgroup path), and the launch (extra = that
// part of the workspace).
size_t select_ws_bytes(int B, int T_q, int64_t q_pos0);
hipError_t launch_select(const SelectArgs &a, void *extra, hipStream_t st);
struct OverlapArgs {
    int B, T_q, top_k;
    const int32_t *a;         // [B][T_q][top_k] ascending, -1 padded
    int64_t a_sb, a_st;
    const int32_t *b;
    int64_t b_sb, b_st;
    int32_t *counts;          // [B * T_q]
};

// Launches the attention kernel and, for a split call, its merge -- unless
// `defer` is set: then the merge is left to the caller (MergeArgs of this
// call in *defer), who hands it to a later launch's `mg` or to launch_merge.
hipError_t launch_attn(const AttnArgs &a, hipStream_t st, MergeArgs *defer = nullptr);
hipError_t launch_merge(const MergeArgs &m, hipStream_t st);
hipError_t launch_overlap(const OverlapArgs &a, hipStream_t st);

}  // namespace lcsi
