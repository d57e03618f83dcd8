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
// Tile: 256 rows x 256 output columns per workgroup of 8 waves, each wave owning 128 rows x 64
// columns (8 x 4 MFMA tiles of 16 x 16).  Columns past the last multiple of 256 go to a second
// launch of 64 x 64 tiles (four waves of 16 rows x 64 columns), so that a remainder such as the
// 64 gate columns of an 8,256-wide in-projection costs a small launch instead of a fifth round
// of whole tiles.  Its K steps are too short to hide a copy behind one step of products, so it
// keeps four K steps in LDS and its copies run three steps ahead.  Both tiles run the same
// MFMA over the same K blocks for every element, so they give the same bits.  K advances in steps of 64, double-buffered in LDS; the next step's
// tiles are copied from global memory straight into LDS (no registers) while the current one
// is multiplied.  The MFMA computes D = W X^T (16 output columns x 16 rows), so that a lane
// holds four adjacent output columns of one row and stores them with one 8- or 16-byte store.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BK = 64, CH = BK / 8;  // CH 16-byte chunks per tile row
constexpr int kThreads = 512;

// 16-byte chunk c of row r of an LDS tile (rows of 128 bytes): the chunk index is XORed with
// (r / 2) mod 8, so the 16 rows a fragment read touches spread over all banks.
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

typedef __attribute__((address_space(3))) void lds_void;

// One ROWS-row x 64-K tile of a row-major [rows][ld] bf16 matrix, rows from r0, copied from
// global memory into the LDS tile L by direct-to-LDS loads.  Each wave instruction fills 1 KB of
// LDS in lane order, so lane i of instruction j fills position p = 64 (J wave + j) + i, and
// fetches the chunk that the swizzle puts there.  Rows at or past `rows` repeat the last row:
// they only feed outputs that are never stored.
template <int ROWS, int NW = 8>
__device__ __forceinline__ void tile_to_lds(const uint16_t *M, int64_t rows, int64_t ld, int64_t r0,
                                            int k0, u32x4 *L, int wave, int lane)
{
    constexpr int J = ROWS * CH / (64 * NW);  // wave instructions per wave (NW waves)
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int p = 64 * (J * wave + j) + lane, r = p / CH, c = (p % CH) ^ ((r >> 1) & 7);
        const int64_t gr = r0 + r < rows ? r0 + r : rows - 1;
        __builtin_amdgcn_global_load_lds((const void *)(M + gr * ld + k0 + 8 * c),
                                         (lds_void *)(L + 64 * (J * wave + j)), 16, 0, 0);
    }
}

// y[:, 0 .. N) (row stride ldy) of a BM x BN tile grid (BN = 256).
template <typename Out, int BN>
__global__ __launch_bounds__(kThreads) void linear_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w,
                                                          Out *__restrict__ y, int64_t T, int K,
                                                          int N, int64_t ldy)
{
    constexpr int NWN = BN / 64, NWM = 8 / NWN;  // waves along N and along M
    constexpr int WM = BM / NWM, RT = WM / 16;   // rows per wave, 16-row MFMA tiles per wave
    // two separate buffers (not one array indexed by parity): the compiler then sees that the
    // copies into one do not alias the reads of the other, and does not wait for them early
    __shared__ u32x4 X0[BM * CH], W0[BN * CH], X1[BM * CH], W1[BN * CH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % NWM, wn = wave / NWM;  // this wave's WM x 64 part
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;
    const int li = lane % 16, kg = lane / 16;

    f32x4 acc[4][RT];  // [output column tile i][row tile j]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < RT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mma = [&](const u32x4 *Xs, const u32x4 *Ws) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8 a[4], b[RT];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = __builtin_bit_cast(bf16x8, Ws[chunk_at(wn * 64 + 16 * i + li, 4 * kb + kg)]);
#pragma unroll
            for (int j = 0; j < RT; ++j)
                b[j] = __builtin_bit_cast(bf16x8, Xs[chunk_at(wm * WM + 16 * j + li, 4 * kb + kg)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < RT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    tile_to_lds<BM>(x, T, K, m0, 0, X0, wave, lane);
    tile_to_lds<BN>(w, N, K, n0, 0, W0, wave, lane);
    __syncthreads();
    const int nk = K / BK;
    for (int kt = 0; kt < nk; kt += 2) {
        // K step kt from buffers 0 while step kt + 1 lands in buffers 1, then the other way
        if (kt + 1 < nk) {
            tile_to_lds<BM>(x, T, K, m0, (kt + 1) * BK, X1, wave, lane);
            tile_to_lds<BN>(w, N, K, n0, (kt + 1) * BK, W1, wave, lane);
        }
        mma(X0, W0);
        __syncthreads();
        if (kt + 1 < nk) {
            if (kt + 2 < nk) {
                tile_to_lds<BM>(x, T, K, m0, (kt + 2) * BK, X0, wave, lane);
                tile_to_lds<BN>(w, N, K, n0, (kt + 2) * BK, W0, wave, lane);
            }
            mma(X1, W1);
            __syncthreads();
        }
    }
    // lane holds D[4 kg + e][li] of each tile: output columns n .. n+3 of row m
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        const int64_t m = m0 + wm * WM + 16 * j + li;
        if (m >= T) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + wn * 64 + 16 * i + 4 * kg;
            if (n < N) store4<Out>(y + m * ldy + n, acc[i][j]);
        }
    }
}

// The column remainder: 64 x 64 tiles of y[:, 0 .. N) (row stride ldy), four waves each
// owning 16 rows x 64 columns.  K steps kt live in LDS stage kt mod 4 (four separate arrays per
// operand); the copy of step kt + 3 is issued once every wave has passed the barrier of step
// kt, that is, once all have finished reading step kt - 1 from the stage it reuses.
constexpr int kNarrow = 64, kNarrowThreads = 256, kStageLoads = 4;  // copies per wave per stage

// Wait until at most n of this wave's copies are outstanding (n = 0, 4 or 8; the counter
// decrements in issue order), then meet the other waves.  The copies of a stage are then in
// LDS for every wave.
__device__ __forceinline__ void wait_copies_and_meet(int n)
{
    __builtin_amdgcn_sched_barrier(0);
    if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);       // vmcnt(8)
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <typename Out>
__global__ __launch_bounds__(kNarrowThreads) void linear_narrow_kernel(const uint16_t *__restrict__ x,
                                                                       const uint16_t *__restrict__ w,
                                                                       Out *__restrict__ y, int64_t T,
                                                                       int K, int N, int64_t ldy)
{
    __shared__ u32x4 X0[kNarrow * CH], X1[kNarrow * CH], X2[kNarrow * CH], X3[kNarrow * CH];
    __shared__ u32x4 W0[kNarrow * CH], W1[kNarrow * CH], W2[kNarrow * CH], W3[kNarrow * CH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * kNarrow;
    const int64_t n0 = (int64_t)blockIdx.y * kNarrow;
    const int li = lane % 16, kg = lane / 16;
    const int nk = K / BK;

    f32x4 acc[4];  // [output column tile i] of this wave's 16 rows
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto copy = [&](int kt, u32x4 *Xs, u32x4 *Ws) {
        tile_to_lds<kNarrow, 4>(x, T, K, m0, kt * BK, Xs, wave, lane);
        tile_to_lds<kNarrow, 4>(w, N, K, n0, kt * BK, Ws, wave, lane);
    };
    // step kt: its copies (issued three steps ago) landed.  Its fragments are read before the
    // copy of kt + 3 (into the stage that step kt - 1 read) is issued, so that no wait for LDS
    // data can include that copy.
    auto step = [&](int kt, const u32x4 *Xc, const u32x4 *Wc, u32x4 *Xn, u32x4 *Wn) {
        const int later = nk - 1 - kt;  // steps whose copies were issued after this one's
        wait_copies_and_meet(kStageLoads * (later < 2 ? later : 2));
        bf16x8 a[2][4], b[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[kb][i] = __builtin_bit_cast(bf16x8, Wc[chunk_at(16 * i + li, 4 * kb + kg)]);
            b[kb] = __builtin_bit_cast(bf16x8, Xc[chunk_at(16 * wave + li, 4 * kb + kg)]);
        }
        if (kt + 3 < nk) copy(kt + 3, Xn, Wn);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kb][i], b[kb], acc[i], 0, 0, 0);
    };

    copy(0, X0, W0);
    if (nk > 1) copy(1, X1, W1);
    if (nk > 2) copy(2, X2, W2);
    for (int kt = 0; kt < nk; kt += 4) {
        step(kt, X0, W0, X3, W3);
        if (kt + 1 < nk) step(kt + 1, X1, W1, X0, W0);
        if (kt + 2 < nk) step(kt + 2, X2, W2, X1, W1);
        if (kt + 3 < nk) step(kt + 3, X3, W3, X2, W2);
    }
    // lane holds D[4 kg + e][li] of each tile: output columns n .. n+3 of row m
    const int64_t m = m0 + 16 * wave + li;
    if (m < T) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + 16 * i + 4 * kg;
            if (n < N) store4<Out>(y + m * ldy + n, acc[i]);
        }
    }
}

template <typename Out>
int launch_tiles(int64_t T, int K, int N, const uint16_t *x, const uint16_t *w, Out *y, hipStream_t st)
{
    const int nw = N / 256 * 256;  // columns in whole 256-wide tiles
    if (nw > 0)
        hipLaunchKernelGGL((linear_kernel<Out, 256>), dim3((unsigned)((T + BM - 1) / BM), (unsigned)(nw / 256)),
                           dim3(kThreads), 0, st, x, w, y, T, K, nw, (int64_t)N);
    if (N > nw)
        hipLaunchKernelGGL((linear_narrow_kernel<Out>),
                           dim3((unsigned)((T + kNarrow - 1) / kNarrow), (unsigned)((N - nw + kNarrow - 1) / kNarrow)),
                           dim3(kNarrowThreads), 0, st, x, w + (int64_t)nw * K, y + nw, T, K, N - nw,
                           (int64_t)N);
    return (int)hipGetLastError();
}

}  // namespace

int launch_linear(int64_t T, int K, int N, const void *x, const void *w, void *y, int out_dtype,
                  void *stream)
{
    (void)hipGetLastError();
    if (T == 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    if (out_dtype == GDN_BF16)
        return launch_tiles<uint16_t>(T, K, N, (const uint16_t *)x, (const uint16_t *)w, (uint16_t *)y, st);
    return launch_tiles<float>(T, K, N, (const uint16_t *)x, (const uint16_t *)w, (float *)y, st);
}

}  // namespace gdn
