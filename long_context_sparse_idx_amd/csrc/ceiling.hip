// Measurement helpers (not steps of the method): the practical ceiling of
// the indexer score kernel's matrix-core work on this chip, and of a plain
// streaming read from HBM (the roof of the memory-bound decode kernels).  A loop issues
// the score kernel's instruction stream -- per 32-key block and wave, 16
// v_mfma_f32_32x32x16_bf16 in two accumulator chains (two 32-row tiles of
// (query, head) rows against the block's keys, 8 k-steps of 16 dims) -- at
// the same occupancy (8 waves per workgroup, two per SIMD), on operands
// drawn like the indexer's (the caller passes N(0,1)/8 bf16 values), but
// with nothing else: no ReLU / weight / head-reduction epilogue, no score
// stores, no key traffic from memory.
//   mode 0: B fragments in registers, four blocks' worth, rotated block by
//           block (the operands change every block, as they do when keys
//           stream through).
//   mode 1: B fragments read from two key tiles staged once in LDS (128
//           keys x 128 dims, rows padded by 16 bytes), block by block, with
//           the score kernel's reads.
// Each wave finally stores one float (the sum of its accumulators), so no
// product is dead.  Work per launch: n_wg * 8 waves * blocks * 16 * 32768
// flop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcsi_ceiling.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NWAVE = 8;
constexpr int KS = 8;              // k-steps of 16 dims (128 dims)
constexpr int ROWB = 128 * 2 + 16; // LDS bytes per key row (+16 B pad), as in the score kernel
constexpr int KT = 128;            // keys per LDS tile

__device__ __forceinline__ bf16x8 ld_frag(const uint16_t *p) { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p)); }

template <int MODE>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(2))) void mfma_loop_kernel(
    const uint16_t *data, float *out, int blocks)
{
    // (mode 1 asks for 96 KB of LDS so that, like the score kernel, one
    // workgroup -- two waves per SIMD -- runs per CU)
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[MODE == 1 ? 96 * 1024 : 16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    // A fragments: rows (lane % 32) of two 32-row tiles, 8 dims of group g per k-step
    const uint16_t *qb = data + ((size_t)(blockIdx.x % 64) * NWAVE + wave) * 64 * 128;
    bf16x8 qa[2][KS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int s = 0; s < KS; ++s) qa[rt][s] = ld_frag(qb + (rt * 32 + l32) * 128 + g * 64 + 8 * s);
    const uint16_t *kbase = data + (size_t)64 * NWAVE * 64 * 128;  // keys after the query rows
    f32x16 acc0 = f32x16{0}, acc1 = f32x16{0};
    if constexpr (MODE == 0) {
        bf16x8 bk[4][KS];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int s = 0; s < KS; ++s) bk[j][s] = ld_frag(kbase + (j * 32 + l32) * 128 + g * 64 + 8 * s);
        for (int it = 0; it < blocks; it += 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], bk[j][s], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], bk[j][s], acc1, 0, 0, 0);
                }
        }
    } else {
        // two tiles of 128 keys staged once (rows padded as in the score kernel)
        for (int c = tid; c < 2 * KT * 16; c += NWAVE * 64) {
            const int row = c / 16, part = c % 16;
            *reinterpret_cast<u32x4 *>(tiles + row * ROWB + part * 16) =
                *reinterpret_cast<const u32x4 *>(kbase + (size_t)row * 128 + part * 8);
        }
        __syncthreads();
        for (int it = 0; it < blocks; ++it) {
            const int cb = it & 7;  // block cb of the 8 blocks in the two tiles
            const uint8_t *src = tiles + (cb * 32 + l32) * ROWB + g * 128;
            bf16x8 bk[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) bk[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(src + 16 * s));
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], bk[s], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], bk[s], acc1, 0, 0, 0);
            }
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc0[i] + acc1[i];
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) out[(size_t)blockIdx.x * NWAVE + wave] = sum;
}

// Streaming read: every 16-byte unit of the buffer once (grid-stride, eight
// loads in flight per thread, non-temporal), XOR-reduced to one word per
// thread so no load is dead.
__global__ __launch_bounds__(256) void read_kernel(const u32x4 *p, size_t n16, uint32_t *out)
{
    constexpr int U = 8;
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (size_t)gridDim.x * blockDim.x;
    u32x4 acc{0, 0, 0, 0};
    size_t i = tid;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    out[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

int lcsi_ceiling_read(const void *data, size_t bytes, uint32_t *out, int n_wg, void *stream)
{
    if (!data || !out || n_wg < 1 || bytes < 16 || bytes % 16) return -1;
    if (((uintptr_t)data % 16) || ((uintptr_t)out % 4)) return -5;
    hipLaunchKernelGGL(read_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4 *>(data), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

size_t lcsi_ceiling_data_elems(void) { return (size_t)64 * NWAVE * 64 * 128 + 2 * KT * 128; }

int lcsi_ceiling_mfma(const uint16_t *data, float *out, int n_wg, int blocks, int mode, void *stream)
{
    if (!data || !out || n_wg < 1 || blocks < 4 || blocks % 4 || (mode != 0 && mode != 1)) return -1;
    if (((uintptr_t)data % 16) || ((uintptr_t)out % 4)) return -5;
    hipStream_t s = (hipStream_t)stream;
    if (mode == 0)
        hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(n_wg), dim3(NWAVE * 64), 0, s, data, out, blocks);
    else
        hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(n_wg), dim3(NWAVE * 64), 0, s, data, out, blocks);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
