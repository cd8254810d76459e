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
//   gather  : the 32 KV rows are read once from HBM; the K part is stored
//             row-major in LDS and the V part transposed (V^T[dim][key]) so
//             the PV product can read 8 consecutive keys of one dim at once.
//   S^T     : 16x16x32 bf16 MFMA with K as the A operand (16 keys) and Q^T
//             as B (16 heads), so a lane ends up holding 8 keys of ONE head.
//             The A-row -> key map is chosen so those 8 keys are consecutive
//             (8g .. 8g+7 for lane group g).
//   softmax : online, in fp32 registers, exp2 with the scale folded in.
//   PV      : O^T = V^T P^T: A from LDS V^T, B = the lane's own 8 p values
//             packed to bf16 -- P never leaves registers; O^T's layout keeps
//             one head per lane, matching the softmax state.
// Each wave owns 16 heads and DV/NDS output dims (NDS = 4 / head groups).
#include "device_common.h"
#include "kernels.h"

namespace lcsi {

namespace {

constexpr int TK = 32;           // indices per tile
constexpr int VTROW = TK * 2 + 16;  // LDS bytes per V^T row (+16 B pad)

__device__ __forceinline__ int32_t usable_index(const AttnArgs &a, const int32_t *row, int j, int j_hi, int64_t p)
{
    if (j >= j_hi) return -1;
    const int32_t v = row[j];
    return (v >= 0 && v <= p && v < a.T_kv) ? v : -1;
}

template <int DQK, int DV, int NDS>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a)
{
    constexpr int KROW = DQK * 2 + 16;     // LDS bytes per K row (+16 B pad)
    constexpr int NCK = DQK / 8;           // 16-byte chunks per K row
    constexpr int NCV = DV / 8;            // 16-byte chunks of V per row
    constexpr int QSTEPS = DQK / 32;
    constexpr int NWH = 4 / NDS;           // head groups of 16
    constexpr int DVW = DV / NDS;          // output dims per wave
    constexpr int NDT = DVW / 16;

    __shared__ __attribute__((aligned(16))) uint8_t sk[TK * KROW];
    __shared__ __attribute__((aligned(16))) uint8_t svt[DV * VTROW];
    __shared__ int32_t sidx[2][TK];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int split = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
    const int64_t p = a.q_pos0 + t;
    const int hg = wave % NWH, ds = wave / NWH;
    const int head = hg * 16 + l16;
    const bool head_ok = head < a.H;
    const int j_lo = split * a.split_len;
    const int j_hi = min(a.top_k, j_lo + a.split_len);
    const int ntile = (j_hi - j_lo + TK - 1) / TK;
    const int32_t *irow = a.idx + (int64_t)b * a.idx_sb + (int64_t)t * a.idx_st;
    const uint16_t *kbase = a.k + (int64_t)b * a.k_sb;
    const uint16_t *vbase = a.v + (int64_t)b * a.v_sb;
    const bool shared_kv = a.v == a.k && a.v_st == a.k_st;

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

    if (tid < TK) sidx[0][tid] = usable_index(a, irow, j_lo + tid, j_hi, p);
    __syncthreads();

    for (int it = 0; it < ntile; ++it) {
        const int buf = it & 1;
        // ---- gather the tile: items (chunk c, group of 4 rows rg)
        {
            const int nitems = (shared_kv ? NCK : NCK + NCV) * (TK / 4);
            for (int item = tid; item < nitems; item += 256) {
                const int c = item >> 3, rg = item & 7;
                const bool kpart = c < NCK;
                const int cc = kpart ? c : c - NCK;      // chunk within its tensor
                const uint16_t *src = kpart ? kbase : vbase;
                const int64_t sst = kpart ? a.k_st : a.v_st;
                u32x4 v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t key = sidx[buf][4 * rg + i];
                    v[i] = key >= 0 ? ld16(src + (int64_t)key * sst + 8 * cc) : u32x4{0, 0, 0, 0};
                }
                if (kpart) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) st16(sk + (4 * rg + i) * KROW + 16 * cc, v[i]);
                }
                const bool vpart = shared_kv ? (kpart && cc < NCV) : !kpart;
                if (vpart) {
                    // transpose 4 rows x 8 dims -> 8 dims x 4 rows
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const uint32_t x0 = v[0][m], x1 = v[1][m], x2 = v[2][m], x3 = v[3][m];
                        const u32x2 lo{(x0 & 0xFFFFu) | (x1 << 16), (x2 & 0xFFFFu) | (x3 << 16)};
                        const u32x2 hi{(x0 >> 16) | (x1 & 0xFFFF0000u), (x2 >> 16) | (x3 & 0xFFFF0000u)};
                        *reinterpret_cast<u32x2 *>(svt + (8 * cc + 2 * m) * VTROW + 8 * rg) = lo;
                        *reinterpret_cast<u32x2 *>(svt + (8 * cc + 2 * m + 1) * VTROW + 8 * rg) = hi;
                    }
                }
            }
        }
        if (tid < TK && it + 1 < ntile) sidx[buf ^ 1][tid] = usable_index(a, irow, j_lo + (it + 1) * TK + tid, j_hi, p);
        const int any = __syncthreads_or(tid < TK && sidx[buf][tid] >= 0);
        if (any) {
            // ---- S^T = K Q^T for 32 keys (two 16-key halves)
            f32x4 sacc[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int krow = 8 * (l16 >> 2) + 4 * hf + (l16 & 3);
                const uint8_t *kp = sk + krow * KROW + 16 * g;
                f32x4 acc{0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < QSTEPS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const u32x4 *>(kp + 64 * s)),
                                                                  qf[s], acc, 0, 0, 0);
                sacc[hf] = acc;
            }
            // ---- online softmax over this lane's keys 8g .. 8g+7 (head l16)
            float sv[8];
            float mt = -__builtin_inff();
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool ok = sidx[buf][8 * g + e] >= 0;
                sv[e] = ok ? sacc[e >> 2][e & 3] * a.sm_scale_log2 : -__builtin_inff();
                mt = fmaxf(mt, sv[e]);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            float pv[8];
            float alpha = 1.f, psum = 0.f;
            if (m_new == -__builtin_inff()) {
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = 0.f;
            } else {
                alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = __builtin_amdgcn_exp2f(sv[e] - m_new);
                    psum += pv[e];
                }
            }
            m_run = m_new;
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int i = 0; i < NDT; ++i) oacc[i] *= alpha;
            const bf16x8 pf = as_bf16x8(u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                              pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});
            // ---- O^T += V^T P^T
            const uint8_t *vp = svt + (ds * DVW + l16) * VTROW + 16 * g;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(*reinterpret_cast<const u32x4 *>(vp + dt * 16 * VTROW)), pf, oacc[dt], 0, 0, 0);
        }
        __syncthreads();
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
        const int64_t row = ((int64_t)b * a.T_q + t) * a.splits + split;
        float *po = a.part_o + (row * a.H + head) * DV + ds * DVW + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(po + dt * 16) = oacc[dt];
        if (ds == 0 && g == 0) {
            float *pm = a.part_ml + (row * a.H + head) * 2;
            pm[0] = m_run;
            pm[1] = l_tot;
        }
    }
}

// Combine the per-split partial results of one query row:
// O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),  M = max_s m_s.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a)
{
    const int64_t row = blockIdx.x;  // b * T_q + t
    const int b = (int)(row / a.T_q), t = (int)(row % a.T_q);
    const int nq = a.DV / 4;
    for (int item = threadIdx.x; item < a.H * nq; item += 256) {
        const int h = item / nq, d = (item % nq) * 4;
        float M = -__builtin_inff();
        for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[((row * a.splits + s) * a.H + h) * 2]);
        f32x4 o{0, 0, 0, 0};
        float L = 0.f;
        if (M != -__builtin_inff()) {
            for (int s = 0; s < a.splits; ++s) {
                const int64_t r = (row * a.splits + s) * a.H + h;
                const float ms = a.part_ml[r * 2];
                if (ms == -__builtin_inff()) continue;
                const float f = __builtin_amdgcn_exp2f(ms - M);
                L += a.part_ml[r * 2 + 1] * f;
                o += *reinterpret_cast<const f32x4 *>(a.part_o + r * a.DV + d) * f;
            }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        o *= inv;
        uint16_t *op = a.out + (int64_t)b * a.o_sb + (int64_t)t * a.o_st + (int64_t)h * a.o_sh + d;
        *reinterpret_cast<u32x2 *>(op) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
}

template <int DQK, int DV>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t st)
{
    dim3 grid(a.splits, a.T_q, a.B);
    const int nwh = (a.H + 15) / 16;
    if (nwh == 1)
        hipLaunchKernelGGL((attn_kernel<DQK, DV, 4>), grid, dim3(256), 0, st, a);
    else if (nwh == 2)
        hipLaunchKernelGGL((attn_kernel<DQK, DV, 2>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((attn_kernel<DQK, DV, 1>), grid, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.B * a.T_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

void attn_plan(int B, int T_q, int top_k, int &splits, int &split_len)
{
    const int64_t rows = (int64_t)B * T_q;
    const int tiles = (top_k + TK - 1) / TK;
    int s = 1;
    if (rows < 256) {
        s = (int)((256 + rows - 1) / rows);
        const int max_s = (tiles + 1) / 2;  // keep >= 2 tiles per split
        if (s > max_s) s = max_s;
        if (s < 1) s = 1;
    }
    const int per = (tiles + s - 1) / s;
    split_len = per * TK;
    splits = (top_k + split_len - 1) / split_len;
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t st)
{
    if (a.DQK == 576 && a.DV == 512) return launch_attn_d<576, 512>(a, st);
    if (a.DQK == 128 && a.DV == 128) return launch_attn_d<128, 128>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace lcsi
