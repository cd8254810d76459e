// Sparse gather attention for gfx950: every query head attends to only the
// rows its index set lists (IndexShare explainer (yun88.com), section on the
// hidden indexer cost: attention restricted to the top-k positions; section
// on the sharing mechanism: every layer, F or S, runs its own attention on
// the set it is given).
//
//   O[b,t,h,:] = sum_j softmax_j(tau * Q[b,t,h,:] . K[b,i_j,:]) V[b,i_j,:]
//
// over the usable entries i_j of the row's index list.  All heads share one
// KV head (MQA), so the heads form the MFMA dimension of one query row.
//
// One workgroup (4 waves) = one query row (and one split of its index list
// when few rows are present).  Per tile of 32 indices:
//   gather  : the 32 KV rows go straight from HBM into LDS with direct
//             global->LDS loads (no staging registers), one tile ahead of the
//             compute, into a double-buffered row-major tile; one gathered
//             row serves as both K and V when V is the first D_v columns of
//             the K row.
//   S^T     : 16x16x32 bf16 MFMA with K as the A operand (16 keys) and Q^T
//             as B (16 heads), so a lane ends up holding 8 keys of ONE head.
//             The A-row -> key map is chosen so those 8 keys are consecutive
//             (8g .. 8g+7 for lane group g).  The two waves of a head group
//             that own neighbouring output-dim slices each compute one
//             16-key half and swap halves through LDS, so K is read from LDS
//             and multiplied once per pair, not once per wave.
//   softmax : online, in fp32 registers, exp2 with the scale folded in.
//   PV      : O^T = V^T P^T: the A operand (8 consecutive keys of one V
//             column) comes from the row-major tile through LDS transpose
//             reads; B = the lane's own 8 p values packed to bf16 -- P never
//             leaves registers; O^T's layout keeps one head per lane,
//             matching the softmax state.
// Each wave owns 16 heads and DV/NDS output dims; a workgroup has NWH head
// groups x NDS dim slices = 4 waves for up to 32 heads, 8 waves for 64 heads
// (so every variant keeps two waves per SIMD resident).
// Decode calls split each row's index list; the parts are merged by
// log-sum-exp either by a merge launch or (MG) by the workgroups of a later
// attention launch, as a prologue whose loads are in flight together with
// the first gather.
#include "device_common.h"
#include "kernels.h"

namespace lcsi {

namespace {

constexpr int TK = 32;  // indices per tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int32_t usable_index(const AttnArgs &a, const int32_t *row, int j, int j_hi, int64_t p)
{
    if (j >= j_hi) return -1;
    const int32_t v = row[j];
    return (v >= 0 && v <= p && v < a.T_kv) ? v : -1;
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i names 8 bytes M[i][0..3] (four b16 values) and lane j receives
// M[4e + j/4][j%4] for e = 0..3.  With lane i pointing at row kb + i/4,
// columns db + 4(i%4) of a row-major tile, lane j gets column db + j of rows
// kb .. kb+3.
// (The builtin is only spelled out for the device pass: in the host pass of
// the same source an LDS builtin on a computed pointer suppresses the
// host-side launch stub of the kernel that calls it, and a __device__
// function never runs on the host.)
__device__ __forceinline__ uint2 lds_read_tr(const uint8_t *p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(const_cast<uint8_t *>(p)));
    return __builtin_bit_cast(uint2, v);
#else
    (void)p;
    return uint2{0, 0};
#endif
}

// max(x[l], x[l ^ 16], x[l ^ 32], x[l ^ 48]) in every lane, with the gfx950
// row-swap VALU ops (no LDS): with both operands x, v_permlane16_swap
// returns x of rows (0,0,2,2) and (1,1,3,3) -- their max is the max over
// the row pair -- and v_permlane32_swap likewise across the two halves.
__device__ __forceinline__ float max_lane_rows(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float m = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const uint32_t v = __float_as_uint(m);
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// ---- Merge of a split call's parts.  With each part's normalised output
// N_s = O_s / l_s (fp16) and its (m_s, l_s) (fp32, log2 units),
//   O = sum_s w_s N_s / sum_s w_s,  w_s = l_s 2^(m_s - M),  M = max_s m_s,
// summed over s in ascending order; parts with no usable key (m_s = -inf)
// are skipped, and a row with none at all gets zeros.  One thread merges NE
// consecutive output dims of one (row, head); every thread of every merging
// kernel does the same arithmetic per element, so the result does not depend
// on which launch merges.
constexpr int MAXS = 8;  // parts of a decode row: at most 2048 / 256

template <int NE>
struct MergeLd {
    uint32_t o[MAXS][NE / 2];
    f32x2 ml[MAXS];
};

// Every part's loads first (parts past S re-read the last one; they are not used).
template <int NE>
__device__ __forceinline__ void merge_load(const MergeArgs &m, int64_t row, int h, int d, MergeLd<NE> &x)
{
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
        const int se = s < m.S ? s : m.S - 1;
        const int64_t r = (row * m.S + se) * m.H + h;
        x.ml[s] = *reinterpret_cast<const f32x2 *>(m.part_ml + r * 2);
        const uint16_t *po = m.part_o + r * m.DV + d;
        if constexpr (NE == 8) {
            const u32x4 v = ld16(po);
#pragma unroll
            for (int i = 0; i < 4; ++i) x.o[s][i] = v[i];
        } else {
            static_assert(NE == 4, "4 or 8 dims per thread");
            const u32x2 v = *reinterpret_cast<const u32x2 *>(po);
            x.o[s][0] = v[0];
            x.o[s][1] = v[1];
        }
    }
}

template <int NE>
__device__ __forceinline__ void merge_store(const MergeArgs &m, int64_t row, int h, int d, const MergeLd<NE> &x)
{
    float M = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
        if (s < m.S) M = fmaxf(M, x.ml[s][0]);
    float o[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] = 0.f;
    float L = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            if (s >= m.S || x.ml[s][0] == -__builtin_inff()) continue;
            const float w = x.ml[s][1] * __builtin_amdgcn_exp2f(x.ml[s][0] - M);
            L += w;
#pragma unroll
            for (int e = 0; e < NE; e += 2) {
                o[e] = __builtin_fmaf(f16_lo(x.o[s][e / 2]), w, o[e]);
                o[e + 1] = __builtin_fmaf(f16_hi(x.o[s][e / 2]), w, o[e + 1]);
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int b = (int)(row / m.T_q), t = (int)(row % m.T_q);
    uint16_t *op = m.out + (int64_t)b * m.o_sb + (int64_t)t * m.o_st + (int64_t)h * m.o_sh + d;
    if constexpr (NE == 8)
        st16(op, u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                       pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)});
    else
        *reinterpret_cast<u32x2 *>(op) = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
}

// The share of merge items (row, head) of one workgroup of a launch that
// hosts another call's merge: items are dealt to the launch's workgroups in
// contiguous runs; within a workgroup, DV/8 threads merge one item (8 dims
// each, 16-byte loads), NT threads take NT/(DV/8) items per pass.
struct MergeShare {
    int64_t it0, it_end;  // this workgroup's items
    int ipp, sub, d;      // items per pass; this thread's item in a pass, its first dim
};

template <int NT>
__device__ __forceinline__ MergeShare merge_share(const MergeArgs &m)
{
    MergeShare sh;
    const int64_t items = (int64_t)m.rows * m.H;
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
    const int64_t wid = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t per = (items + nwg - 1) / nwg;
    sh.it0 = wid * per;
    sh.it_end = min(items, sh.it0 + per);
    const int tpi = m.DV / 8;
    sh.ipp = NT / tpi;
    sh.sub = (int)threadIdx.x / tpi;
    sh.d = 8 * ((int)threadIdx.x % tpi);
    return sh;
}

template <int DQK, int DV, int NWH, int NDS, bool SHARED, bool MG>
__global__ __launch_bounds__(64 * NWH * NDS) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(AttnArgs a)
{
    // Row-major KV tile in LDS: each row holds the K row (DQK bf16) and, when
    // V is a separate tensor, the V row after it, plus one 16-byte pad slot.
    constexpr int NCK = DQK / 8;                      // 16-byte chunks of a K row
    constexpr int NCV = SHARED ? 0 : DV / 8;          // chunks of a separate V row
    constexpr int RS = NCK + NCV + 1;                 // 16-byte slots per LDS row
    constexpr int ROWB = RS * 16;
    constexpr int VOFF = SHARED ? 0 : DQK * 2;        // byte offset of V within a row
    constexpr int NDMA = (TK * RS + 63) / 64;         // 1 KB direct loads per tile
    constexpr int BUFB = NDMA * 1024;                 // bytes per tile buffer
    constexpr int QSTEPS = DQK / 32;
    constexpr int NW = NWH * NDS;                     // waves per workgroup
    constexpr int DVW = DV / NDS;                     // output dims per wave
    constexpr int NDT = DVW / 16;
    static_assert(NDS % 2 == 0, "the dim-slice waves of a head group work in pairs");

    // Two separately declared buffers, each named at compile time in the
    // unrolled tile loop below: the compiler can then tell that the reads of
    // one buffer do not depend on the direct loads still filling the other,
    // and lets them overlap (with one array indexed by a run-time buffer
    // number it waits for every outstanding direct load before each LDS read).
    __shared__ __attribute__((aligned(1024))) uint8_t kv0[BUFB];
    __shared__ __attribute__((aligned(1024))) uint8_t kv1[BUFB];
    // S^T halves handed between the two waves of a pair (same head group,
    // neighbouring dim slices): each computes 16 of the tile's 32 keys.  One
    // array per half, each named at compile time where it is read, so the
    // compiler can tell these reads from the direct loads still filling the
    // next tile (through one array it waited for all of them first).
    __shared__ f32x4 sxa[NW / 2 * 64];
    __shared__ f32x4 sxb[NW / 2 * 64];

    // (the wave index as a scalar: the LDS destinations of the direct loads
    // built from it are then scalar too)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4,
              l16 = lane & 15;
    // blockIdx.x = split + splits * (head block): when a row's heads are
    // shared out between workgroups (decode), the workgroups that gather the
    // same rows of one split sit `splits` apart in launch order, so with
    // 8 splits they land on the same XCD (workgroups go round-robin over the
    // 8 XCDs) and the second gather of a row hits that XCD's L2.
    const int split = blockIdx.x % a.splits, hblk = blockIdx.x / a.splits, t = blockIdx.y, b = blockIdx.z;
    const int64_t p = a.q_pos0 + t;
    const int hg = wave % NWH, ds = wave / NWH;
    const int hf = ds & 1, pr = hg + NWH * (ds >> 1);  // half of S^T this wave computes; its pair
    const int head = (hblk * NWH + hg) * 16 + l16;
    const bool head_ok = head < a.H;
    const int j_lo = split * a.split_len;
    const int j_hi = min(a.top_k, j_lo + a.split_len);
    const int ntile = (j_hi - j_lo + TK - 1) / TK;
    const int32_t *irow = a.idx + (int64_t)b * a.idx_sb + (int64_t)t * a.idx_st;
    const uint16_t *kbase = a.k + (int64_t)b * a.k_sb;
    const uint16_t *vbase = a.v + (int64_t)b * a.v_sb;

    // Q^T fragments (B operand): head l16 of this wave's group, 8 dims of group g per k-step
    bf16x8 qf[QSTEPS];
    {
        const uint16_t *qp = a.q + (int64_t)b * a.q_sb + (int64_t)t * a.q_st + (int64_t)head * a.q_sh + 8 * g;
#pragma unroll
        for (int s = 0; s < QSTEPS; ++s) qf[s] = as_bf16x8(head_ok ? ld16(qp + 32 * s) : u32x4{0, 0, 0, 0});
    }

    f32x4 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0, 0, 0, 0};
    float m_run = -__builtin_inff(), l_run = 0.f;

    // ---- index handling: lanes l and l+32 of every wave hold entry l of a
    // tile's index list (usable index or -1).  The raw entries of tile it+2
    // are loaded while tile it computes, so no load waits on them.
    auto raw_idx = [&](int tile) -> int32_t {
        const int j = j_lo + tile * TK + (lane & 31);
        return (tile < ntile && j < j_hi) ? irow[j] : -1;
    };
    auto usable = [&](int32_t v) -> int32_t { return (v >= 0 && v <= p && v < a.T_kv) ? v : -1; };
    // ---- gather: direct global->LDS loads of one tile (wave w issues loads
    // w, w+NW, ...; lane l of load m fills 16-byte slot 64m + l, which is
    // chunk c of tile row r).  Unusable indices read row 0 instead (finite
    // data; their keys are masked), pad slots and slots past the tile
    // re-read the row's first chunk.
    // The slot -> (tile row, source, byte offset) map of this lane's loads is
    // the same for every tile: worked out once here.
    constexpr int MPW = (NDMA + NW - 1) / NW;  // direct loads per wave and tile
    int g_row[MPW];
    uint32_t g_off[MPW];
    bool g_v[MPW];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
        const int slot = 64 * (wave + NW * i) + lane;
        const int row = slot / RS, c = slot - row * RS;
        g_row[i] = row < TK ? row : 0;
        g_v[i] = c >= NCK && c < NCK + NCV;
        g_off[i] = c < NCK ? 16 * c : (g_v[i] ? 16 * (c - NCK) : 0);
    }
    const uint8_t *kb8 = reinterpret_cast<const uint8_t *>(kbase);
    const uint8_t *vb8 = reinterpret_cast<const uint8_t *>(vbase);
    // row strides in bytes (below 4 GiB, checked on the host)
    const uint32_t kst_b = (uint32_t)(a.k_st * 2), vst_b = (uint32_t)(a.v_st * 2);
    auto gather = [&](int32_t keys, uint8_t *dst) {
        // every lane's key of every load first (the shuffles go out back to
        // back), then the loads
        uint32_t kr[MPW];
#pragma unroll
        for (int i = 0; i < MPW; ++i) {
            const int32_t key = __shfl(keys, g_row[i]);
            kr[i] = key >= 0 ? (uint32_t)key : 0u;
        }
#pragma unroll
        for (int i = 0; i < MPW; ++i) {
            const int m = wave + NW * i;
            if (m >= NDMA) break;
            const uint8_t *src = (NCV && g_v[i] ? vb8 + (uint64_t)kr[i] * vst_b : kb8 + (uint64_t)kr[i] * kst_b) + g_off[i];
            load_to_lds16(src, dst + 1024 * m);
        }
    };

    const int32_t raw0 = raw_idx(0);
    int32_t raw_next = raw_idx(1);
    // MG: this workgroup's share of an earlier split call's merge.  The first
    // pass's loads go out before the first gather and are used while the
    // gather is in flight; further passes (more items than one pass of the
    // workgroup takes) follow.
    MergeShare msh{};
    MergeLd<8> mld;
    int64_t m_it = 0;
    if constexpr (MG) {
        msh = merge_share<64 * NW>(a.mg);
        m_it = msh.it0 + msh.sub;
        // (loaded unconditionally -- a thread without an item re-reads item
        // 0 and stores nothing -- so no branch makes the compiler wait for
        // these loads before the gather's index shuffles)
        const int64_t li = m_it < msh.it_end ? m_it : 0;
        merge_load<8>(a.mg, li / a.mg.H, (int)(li % a.mg.H), msh.d, mld);
    }
    const int32_t keys0 = usable(raw0);
    gather(keys0, kv0);
    uint32_t vmask = (uint32_t)__ballot(keys0 >= 0);  // bit r: tile row r usable
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (MG) {
        // (stored after the wait above: the first tile's wait does not
        // include these stores)
        if (m_it < msh.it_end) merge_store<8>(a.mg, m_it / a.mg.H, (int)(m_it % a.mg.H), msh.d, mld);
        for (m_it += msh.ipp; m_it - msh.sub < msh.it_end; m_it += msh.ipp) {
            if (m_it >= msh.it_end) continue;
            merge_load<8>(a.mg, m_it / a.mg.H, (int)(m_it % a.mg.H), msh.d, mld);
            merge_store<8>(a.mg, m_it / a.mg.H, (int)(m_it % a.mg.H), msh.d, mld);
        }
    }
    // tile `it` computes from `tb` while tile it+1 is gathered into `nb`
    auto step = [&](int it, const uint8_t *tb, uint8_t *nb) {
        const int32_t keys_next = usable(raw_next);
        raw_next = raw_idx(it + 2);
        if (it + 1 < ntile) gather(keys_next, nb);
        const uint32_t vcur = (vmask >> (8 * g)) & 0xFFu;  // this lane's keys 8g .. 8g+7
        const bool any = vmask != 0;
        if (any) {
            // ---- S^T = K Q^T for 32 keys in two 16-key halves: this wave
            // computes half hf -- as two interleaved MFMA chains over the even
            // and odd k-steps -- and takes the other from its partner wave
            // through LDS (the waves of a pair hold the same heads, so lane l
            // of both holds the same (head, key) slots).  Lane (g, head) then
            // holds keys 8g + 4hf + r (own, r < 4) and 8g + 4(1 - hf) + r
            // (other); this wave keeps them in that order as its 8 softmax
            // values and PV k-slots, and reads V's rows in the same order.
            const uint8_t *kp = tb + (8 * (l16 >> 2) + (l16 & 3) + 4 * hf) * ROWB + 16 * g;
            f32x4 c0 = f32x4{0, 0, 0, 0}, c1 = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < QSTEPS; s += 2) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const u32x4 *>(kp + 64 * s)),
                                                             qf[s], c0, 0, 0, 0);
                if (s + 1 < QSTEPS)
                    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(*reinterpret_cast<const u32x4 *>(kp + 64 * (s + 1))), qf[s + 1], c1, 0, 0, 0);
            }
            const f32x4 own = c0 + c1;
            if (hf)
                sxb[pr * 64 + lane] = own;
            else
                sxa[pr * 64 + lane] = own;
            wait_lgkmcnt0();  // (the next tile's direct loads stay in flight)
            lds_barrier();
            const f32x4 other = hf ? sxa[pr * 64 + lane] : sxb[pr * 64 + lane];
            // ---- online softmax over this lane's 8 keys (head l16), in
            // log2 units: logit = sm_scale_log2 * s (sm_scale_log2 > 0, so the
            // maximum of the raw scores gives the maximum logit)
            float sr[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sr[r] = own[r];
                sr[4 + r] = other[r];
            }
            if (__builtin_expect(vmask != 0xFFFFFFFFu, 0)) {  // (tile-uniform: only tiles with unusable entries)
                const uint32_t vk = ((vcur >> (4 * hf)) & 0xFu) | (((vcur >> (4 - 4 * hf)) & 0xFu) << 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!((vk >> e) & 1u)) sr[e] = -__builtin_inff();
            }
            float mt = fmaxf(fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3])), fmaxf(fmaxf(sr[4], sr[5]), fmaxf(sr[6], sr[7])));
            mt = max_lane_rows(mt) * a.sm_scale_log2;  // over the 4 lane groups: the head's 32 keys
            // The reference m_run of the exponentials moves only when the
            // tile's maximum exceeds it by more than 8 (log2 units): the
            // p values then stay below 2^8 (exact range for bf16 and fp32),
            // and O and l are rescaled only on such a move, not on every
            // new maximum (O / l is the same for any reference).
            const bool bump = mt > m_run + 8.f;  // (from -inf: any usable key)
            const float m_new = bump ? mt : m_run;
            // (while no key of the head was usable, every logit is -inf and
            // p = 2^-inf = 0 against any finite reference)
            const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
            const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            float pv[8];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[e], a.sm_scale_log2, -m_use));
                psum += pv[e];
            }
            m_run = m_new;
            l_run = l_run * alpha + psum;
            if (__ballot(bump)) {
#pragma unroll
                for (int i = 0; i < NDT; ++i) oacc[i] *= alpha;
            }
            const bf16x8 pfv = as_bf16x8(u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                               pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});
            // ---- O^T += V^T P^T; A = column (ds*DVW + dt*16 + l16) of this
            // wave's 8 keys in its order: rows 8g + 4hf .. +3, then the other 4
            const uint8_t *vp = tb + (8 * g + 4 * hf + (l16 >> 2)) * ROWB + VOFF + 2 * (ds * DVW + 4 * (l16 & 3));
            const int vo = hf ? -4 * ROWB : 4 * ROWB;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const uint2 lo = lds_read_tr(vp + 32 * dt);
                const uint2 hi = lds_read_tr(vp + vo + 32 * dt);
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}), pfv,
                                                                   oacc[dt], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into the other buffer have landed
        __syncthreads();
        vmask = (uint32_t)__ballot(keys_next >= 0);
    };
    for (int it = 0; it < ntile; it += 2) {
        step(it, kv0, kv1);
        if (it + 1 >= ntile) break;
        step(it + 1, kv1, kv0);
    }

    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!head_ok) return;
    if (a.splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *op = a.out + (int64_t)b * a.o_sb + (int64_t)t * a.o_st + (int64_t)head * a.o_sh + ds * DVW + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const f32x4 o = oacc[dt] * inv;
            *reinterpret_cast<u32x2 *>(op + dt * 16) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
    } else {
        // the part's own normalised output O / l in fp16 (a convex
        // combination of V rows, so within fp16's range; 11 significant
        // bits, more than the bf16 result keeps), and (m, l) in fp32
        const int64_t row = ((int64_t)b * a.T_q + t) * a.splits + split;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *po = a.part_o + (row * a.H + head) * DV + ds * DVW + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const f32x4 o = oacc[dt] * inv;
            *reinterpret_cast<u32x2 *>(po + dt * 16) = u32x2{pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3])};
        }
        if (ds == 0 && g == 0) {
            float *pm = a.part_ml + (row * a.H + head) * 2;
            pm[0] = m_run;
            pm[1] = l_tot;
        }
    }
}

// The merge as a launch of its own: one workgroup per (head, row), thread i
// merges output dims 4i .. 4i+3.
__global__ __launch_bounds__(128) void attn_merge_kernel(MergeArgs m)
{
    const int h = blockIdx.x;
    const int64_t row = blockIdx.y;  // b * T_q + t
    const int d = 4 * threadIdx.x;
    if (d >= m.DV) return;
    MergeLd<4> x;
    merge_load<4>(m, row, h, d, x);
    merge_store<4>(m, row, h, d, x);
}

template <int DQK, int DV, bool SHARED, bool MG>
hipError_t launch_attn_k(const AttnArgs &a, hipStream_t st)
{
    dim3 grid(a.splits * a.hgroups, a.T_q, a.B);
    const int nwh = ((a.H + 15) / 16 + a.hgroups - 1) / a.hgroups;  // 16-head groups per workgroup
    if (a.hgroups > 1) {
        // heads shared out between workgroups: two dim slices per head
        // group, as in the one-workgroup kernels for more than 16 heads, so
        // every head sees exactly the same arithmetic
        if (nwh == 1) {
            // (not planned for separate 576/512 K and V rows: a wave's share
            // of the gather map would spill)
            if constexpr (SHARED || DQK != 576)
                hipLaunchKernelGGL((attn_kernel<DQK, DV, 1, 2, SHARED, MG>), grid, dim3(128), 0, st, a);
            else
                return hipErrorInvalidValue;
        } else {
            hipLaunchKernelGGL((attn_kernel<DQK, DV, 2, 2, SHARED, MG>), grid, dim3(256), 0, st, a);
        }
    } else if (nwh == 1) {
        hipLaunchKernelGGL((attn_kernel<DQK, DV, 1, 4, SHARED, MG>), grid, dim3(256), 0, st, a);
    } else if (nwh == 2) {
        hipLaunchKernelGGL((attn_kernel<DQK, DV, 2, 2, SHARED, MG>), grid, dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL((attn_kernel<DQK, DV, 4, 2, SHARED, MG>), grid, dim3(512), 0, st, a);
    }
    return hipGetLastError();
}

template <int DQK, int DV, bool SHARED>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t st, MergeArgs *defer)
{
    hipError_t e = a.mg.S > 1 ? launch_attn_k<DQK, DV, SHARED, true>(a, st) : launch_attn_k<DQK, DV, SHARED, false>(a, st);
    if (e != hipSuccess || a.splits == 1) return e;
    MergeArgs m{};
    m.part_o = a.part_o;
    m.part_ml = a.part_ml;
    m.out = a.out;
    m.o_sb = a.o_sb;
    m.o_st = a.o_st;
    m.o_sh = a.o_sh;
    m.rows = a.B * a.T_q;
    m.T_q = a.T_q;
    m.H = a.H;
    m.DV = a.DV;
    m.S = a.splits;
    if (defer) {
        *defer = m;
        return hipSuccess;
    }
    return launch_merge(m, st);
}

}  // namespace

#ifndef ATTN_DECODE_TILES
#define ATTN_DECODE_TILES 8     // index tiles per split of a decode row
#endif
#ifndef ATTN_WG_TARGET
// Workgroups a decode call aims for by sharing out heads.  Every workgroup
// sharing a row's heads gathers the row's KV rows again (from L2 at best),
// which costs more than leaving CUs idle, down to about half the chip
// (kernel traces, one machine per comparison): at 32 rows x 8 parts one
// 64-head workgroup per part (256 workgroups) beat two 32-head ones (512),
// 31.9-32.3 vs 32.8-33.4 us per decode131k layer; at 8 rows x 8 parts two
// 32-head workgroups per part (128) beat four 16-head ones (256) and one
// 64-head one (64): 21.0-21.4 vs 22.9-23.4 and 26.9 us per decode1m layer.
#define ATTN_WG_TARGET 128
#endif

AttnPlan attn_plan(int B, int T_q, int H, int DQK, int top_k)
{
    (void)DQK;
    AttnPlan pl{1, 0};
    const int tiles = (top_k + TK - 1) / TK;
    // A decode call (one query row per sequence) splits every row's index
    // list into parts of ATTN_DECODE_TILES tiles, merged by log-sum-exp; a
    // multi-row call runs each row in one workgroup.  Either way the parts
    // -- and so the bits of the result -- are fixed by top_k alone for that
    // kind of call, whatever B is.
    const int s = T_q == 1 ? (tiles + ATTN_DECODE_TILES - 1) / ATTN_DECODE_TILES : 1;
    const int per = (tiles + s - 1) / s;
    pl.split_len = per * TK;
    pl.splits = (top_k + pl.split_len - 1) / pl.split_len;
    (void)B;
    (void)H;
    return pl;
}

hipError_t launch_merge(const MergeArgs &m, hipStream_t st)
{
    if (m.S < 2 || m.S > MAXS || !(m.DV == 512 || m.DV == 128)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(m.H, m.rows), dim3(128), 0, st, m);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a_in, hipStream_t st, MergeArgs *defer)
{
    AttnArgs a = a_in;
    // one gathered row serves K and V when V is the first D_v columns of the
    // same rows, batch entry by batch entry
    const bool shared = a.v == a.k && a.v_st == a.k_st && (a.v_sb == a.k_sb || a.B == 1);
    // few rows (decode): share each row's heads out between workgroups -- no
    // change to any head's arithmetic -- until the call has enough
    // workgroups.  One head group per workgroup (two waves) only where a
    // wave's gather map fits its registers: a shared KV row, or 128-wide rows.
    a.hgroups = 1;
    if (a.T_q == 1 && a.H > 16) {
        const int hb = (a.H + 15) / 16;
        const int gmax = (shared || a.DQK == 128) ? hb : hb / 2;
        const int64_t rows = (int64_t)a.B * a.T_q;
        while (a.hgroups < 4 && 2 * a.hgroups <= gmax && rows * a.splits * a.hgroups < ATTN_WG_TARGET) a.hgroups *= 2;
    }
    if (a.mg.S > 1 && (a.mg.S > MAXS || !(a.mg.DV == 512 || a.mg.DV == 128))) return hipErrorInvalidValue;
    if (a.DQK == 576 && a.DV == 512)
        return shared ? launch_attn_d<576, 512, true>(a, st, defer) : launch_attn_d<576, 512, false>(a, st, defer);
    if (a.DQK == 128 && a.DV == 128)
        return shared ? launch_attn_d<128, 128, true>(a, st, defer) : launch_attn_d<128, 128, false>(a, st, defer);
    return hipErrorInvalidValue;
}

}  // namespace lcsi
