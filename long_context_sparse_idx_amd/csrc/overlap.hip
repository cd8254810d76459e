// Index-set overlap between two layers' top-k lists, the statistic behind
// choosing which layers keep an indexer: adjacent layers pick largely the
// same positions (IndexCache news article (app.myzaker.com), section
// "IndexCache"), and for an existing model the F/S split is searched layer
// by layer, greedily (IndexCache article after VentureBeat
// (linkstar.cloud), section on the two deployment routes).
//
// Per query row: count = |{a_j >= 0} ∩ {b_j >= 0}| for two index lists of
// top_k entries, each ascending with -1 padding at the end (the layout the
// selection writes).  One wave per row: lane l takes a[l], a[l+64], ... and
// binary-searches it in the usable prefix of b.
#include "device_common.h"
#include "kernels.h"

namespace lcsi {

namespace {

constexpr int OV_WAVES = 4;

__global__ __launch_bounds__(OV_WAVES * 64) void overlap_kernel(OverlapArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * OV_WAVES + (threadIdx.x >> 6);
    if (row >= (int64_t)a.B * a.T_q) return;
    const int b = (int)(row / a.T_q), t = (int)(row % a.T_q);
    const int32_t *ra = a.a + b * a.a_sb + (int64_t)t * a.a_st;
    const int32_t *rb = a.b + b * a.b_sb + (int64_t)t * a.b_st;
    // usable length of b: entries before the first -1 (binary search on the
    // sign, the list being ascending with the padding at the end)
    int lo = 0, hi = a.top_k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (rb[mid] >= 0) lo = mid + 1; else hi = mid;
    }
    const int nb = lo;
    int cnt = 0;
    for (int j = lane; j < a.top_k; j += 64) {
        const int32_t x = ra[j];
        if (x < 0) continue;
        int l = 0, h = nb;  // first position in b with value >= x
        while (l < h) {
            const int m = (l + h) >> 1;
            if (rb[m] < x) l = m + 1; else h = m;
        }
        cnt += (l < nb && rb[l] == x);
    }
    cnt = wave_sum_int(cnt);
    if (lane == 0) a.counts[row] = cnt;
}

}  // namespace

hipError_t launch_overlap(const OverlapArgs &a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.B * a.T_q;
    hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)((rows + OV_WAVES - 1) / OV_WAVES)), dim3(OV_WAVES * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcsi
