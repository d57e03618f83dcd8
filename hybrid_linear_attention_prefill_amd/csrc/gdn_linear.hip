// gdn_linear.hip -- the projections around a Gated DeltaNet layer: y = x W^T in bf16 with fp32
// accumulation, on gfx950 MFMA, with one tiling and one K order for every row count.
//
// The pages run the projections of a shared prefix and of every branch with a GEMM handle fixed
// to one algorithm per weight shape, so that a result equals a plain pass over the full prompt
// bit for bit however the prompts are grouped; a library that picks its algorithm by row count
// differs by rounding (PR "qwen3_5: run prompts that share prefixes once per prefix", section
// Purpose, "GEMMs").  Here that holds by construction: every output element is the sum over K
// in the same 32-wide blocks, in the same order, by the same MFMA, whatever the row count, the
// row's place in its tile or the grid; there is no split-K and no shape-dependent choice.
//
// Tile: 128 rows x 128 output columns per workgroup, 4 waves each owning 64 x 64 (4 x 4 MFMA
// tiles of 16 x 16), K in steps of 64 staged in LDS (double-buffered, one barrier per step).
// The MFMA computes D = W X^T (16 output columns x 16 rows), so that a lane holds four adjacent
// output columns of one row and stores them with one 8- or 16-byte store.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64, CH = BK / 8;  // CH 16-byte chunks per tile row

// 16-byte chunk c of row r of an LDS tile: the chunk index is XORed with (r / 2) mod 8, so the
// 16 rows a fragment read touches (and the rows a store wave writes) spread over all banks.
__device__ __forceinline__ int chunk_at(int r, int c) { return r * CH + (c ^ ((r >> 1) & 7)); }

__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

template <typename Out>
__device__ __forceinline__ void store4(Out *p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float *p, f32x4 v)
{
    *(f32x4 *)p = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t *p, f32x4 v)
{
    *(u32x2 *)p = u32x2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
}

// One 128-row x 64-K tile of a row-major [rows][ld] bf16 matrix, rows from r0 (rows at or past
// `rows` read as zero), into registers: 4 chunks per thread.
__device__ __forceinline__ void load_tile(const uint16_t *M, int64_t rows, int64_t ld, int64_t r0,
                                          int k0, int tid, u32x4 (&v)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i, r = id / CH, c = id % CH;
        v[i] = (r0 + r < rows) ? *(const u32x4 *)(M + (r0 + r) * ld + k0 + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_tile(u32x4 *L, int tid, const u32x4 (&v)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        L[chunk_at(id / CH, id % CH)] = v[i];
    }
}

template <typename Out>
__global__ __launch_bounds__(256) void linear_kernel(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ w,
                                                     Out *__restrict__ y, int64_t T, int K, int N)
{
    __shared__ u32x4 Xs[2][BM * CH], Ws[2][BN * CH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;     // this wave's 64 x 64 quarter
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;
    const int li = lane % 16, kg = lane / 16;

    f32x4 acc[4][4];  // [output column tile i][row tile j]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 xv[4], wv[4];
    load_tile(x, T, K, m0, 0, tid, xv);
    load_tile(w, N, K, n0, 0, tid, wv);
    store_tile(Xs[0], tid, xv);
    store_tile(Ws[0], tid, wv);
    __syncthreads();
    const int nk = K / BK;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {  // the next K step, in flight during this one's MFMAs
            load_tile(x, T, K, m0, (kt + 1) * BK, tid, xv);
            load_tile(w, N, K, n0, (kt + 1) * BK, tid, wv);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = __builtin_bit_cast(bf16x8, Ws[buf][chunk_at(wn * 64 + 16 * i + li, 4 * kb + kg)]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = __builtin_bit_cast(bf16x8, Xs[buf][chunk_at(wm * 64 + 16 * j + li, 4 * kb + kg)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            store_tile(Xs[buf ^ 1], tid, xv);
            store_tile(Ws[buf ^ 1], tid, wv);
        }
        __syncthreads();
    }
    // lane holds D[4 kg + e][li] of each tile: output columns n .. n+3 of row m
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 64 + 16 * j + li;
        if (m >= T) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + wn * 64 + 16 * i + 4 * kg;
            if (n < N) store4<Out>(y + m * N + n, acc[i][j]);
        }
    }
}

}  // namespace

int launch_linear(int64_t T, int K, int N, const void *x, const void *w, void *y, int out_dtype,
                  void *stream)
{
    (void)hipGetLastError();
    if (T == 0) return 0;
    const dim3 grid((unsigned)((T + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
    hipStream_t st = (hipStream_t)stream;
    if (out_dtype == GDN_BF16)
        hipLaunchKernelGGL(linear_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)x,
                           (const uint16_t *)w, (uint16_t *)y, T, K, N);
    else
        hipLaunchKernelGGL(linear_kernel<float>, grid, dim3(256), 0, st, (const uint16_t *)x,
                           (const uint16_t *)w, (float *)y, T, K, N);
    return (int)hipGetLastError();
}

}  // namespace gdn
