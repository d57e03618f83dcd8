// gdn_kernels.hip -- HIP kernels for gfx950 (MI355X): chunked Gated DeltaNet prefill.
//
// The layer is the gated delta rule over a width-4 causal conv, run in sub-chunks of 64 rows
// that start at absolute multiples of 64 (the pages keep the fp32 recurrent state and "the
// last three conv inputs" per linear-attention layer: PR "qwen3_5: run prompts that share
// prefixes once per prefix", section Purpose; they require a resumed prefill to equal a fresh
// one bit for bit on the same grid: "The shadow reader", section "Exact on a grid").
//
// Per sub-chunk of n <= 64 rows (K, Q normalised keys/queries, V values, beta, g log decays)
// entered with state S [d_k][d_v]:
//   G_r = sum_{i<=r} g_i;  Gam_ri = exp(G_r - G_i) (i <= r);  gamma_r = exp(G_r)
//   A   = strict_lower(diag(beta) (K K^T) * Gam);  Tinv = (I + A)^-1
//   D   = Tinv diag(beta) (V - diag(gamma) K S)
//   O   = scale (diag(gamma) Q S + (lower(Q K^T) * Gam) D)
//   S'  = gamma_n S + K^T (diag(exp(G_n - G)) D)
// which equals the per-token rule S <- e^g (I - beta k k^T) S + beta k v^T, o = scale S^T q.
// Only exponentials of non-positive differences are formed (G reaches about -52 over 64 rows
// at the usual decays, and e^{-G} alone would overflow fp32).
//
// Kernels, all launched on the caller's stream:
//   prep_kernel    grid (sub-chunks, key heads): conv of the q|k channels, L2 norm, K K^T and
//                  Q K^T on MFMA, and for each value head of the group the cumulative gates,
//                  Tinv (blocked forward substitution in LDS, fp32) and the decayed mask M.
//                  Everything it writes is independent of the state, so all sub-chunks run
//                  in parallel.
//   chain_kernel   grid (d_v tiles of 16, value heads, sequences): the serial walk over the
//                  sub-chunks.  Columns of S evolve independently, so each workgroup owns
//                  S[:, 16 columns] in MFMA accumulators (fp32) for the whole call, with an
//                  fp16 copy in LDS as the MFMA operand.  It also convolves its own v columns.
//   window_kernel  the new conv window = the last 3 rows of (window ++ x), copied bit for bit.
//
// Precision: every MFMA takes fp16 operands (v_mfma_f32_16x16x32_f16, same peak as bf16 on
// gfx950) with fp32 accumulation; all operands are bounded (unit-norm q/k, decays <= 1,
// |Tinv| and |M| of order 1), and fp16's 11-bit significand keeps the operand rounding at
// about 2^-12 relative where bf16 would cost about 2^-9.  The state, gates, conv and norms
// are fp32.
//
// Determinism: every sub-chunk runs the same instruction sequence wherever it falls in a call;
// the only arithmetic boundary is the absolute multiple of 64; the tiling depends only on the
// layer shape; there are no atomics.  So one call over rows [0, N) and any split of it into
// calls at multiples of 64 give identical bits.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "gdn_internal.h"

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                           // nearest even
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t *p, float v) { p->bits = f32_to_bf16_bits(v); }

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c)
{
    // D[m][n] += sum_k A[m][k] B[k][n], 16x16x32.  Lane l supplies A[l%16][8(l/16) .. +7] and
    // B[8(l/16) .. +7][l%16]; it receives D[4(l/16) + i][l%16], i = 0..3.
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef short short4_t __attribute__((ext_vector_type(4)));

// A fragment of K^T for the 16x16x32 MFMA read straight from row-major K in LDS:
// lane (m, kg) of the result holds K[r0 + 8 kg + e][c0 + m], e = 0..7.  ds_read_b64_tr_b16
// hands lane i of each 16-lane group element i % 4 of the 4-element reads of lanes
// 4 e + i / 4, so lane j reads K[row0 + j / 4][c0 + 4 (j % 4) .. + 3] (rows row0 .. row0 + 3).
__device__ __forceinline__ half8 ktrans_frag(const _Float16 *K, int stride, int r0, int c0, int lane)
{
    const int j = lane % 16, kg = lane / 16;
    const _Float16 *p0 = K + (r0 + 8 * kg + j / 4) * stride + c0 + 4 * (j % 4);
    typedef __attribute__((address_space(3))) short4_t lds_short4;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(p0));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(p0 + 4 * stride));
    return __builtin_shufflevector(__builtin_bit_cast(half4, lo), __builtin_bit_cast(half4, hi), 0, 1,
                                   2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ int find_seg(const SegArgs &sa, int sub)
{
    int s = 0;
    for (int i = 1; i < sa.n_seg; ++i)
        if (sa.seg[i].sub0 <= sub) s = i;
    return s;
}

// Packed lower-triangular 64x64 factors (Tinv and M): the 10 tiles (i, j <= i) of 16x16 in
// the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3); inside a tile the
// 256 values sit in MFMA accumulator order: element (r, c) at (r % 4) * 64 + (r / 4) * 16 + c,
// so 16-byte chunk q holds row 4 ((q % 8) / 2) + q / 8, columns (q % 2) * 8 .. + 7.
__device__ __forceinline__ int tile_i(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }
__device__ __forceinline__ int tile_j(int p) { return p - tile_i(p) * (tile_i(p) + 1) / 2; }
__device__ __forceinline__ int chunk_row(int q) { return 4 * ((q % 8) / 2) + q / 8; }
__device__ __forceinline__ int chunk_col(int q) { return (q % 2) * 8; }

template <typename Act>
__device__ __forceinline__ void load8(const u32x4 *row, int cl, float (&v)[8])
{
    if constexpr (sizeof(Act) == 2) {
        const u32x4 u = row[cl / 8];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const u32x4 a = row[cl / 4], b = row[cl / 4 + 1];
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    }
}

// ------------------------------------------------------------------------------------------
// prep_kernel: state-independent factors of one (sub-chunk, key head).
// ------------------------------------------------------------------------------------------
template <int D, typename Act>
__global__ __launch_bounds__(256, 2) void prep_kernel(SegArgs sa, const Act *__restrict__ x,
                                                      const Act *__restrict__ conv_w, int conv_on,
                                                      int silu, const float *__restrict__ g,
                                                      const float *__restrict__ beta, int Hk,
                                                      int Hv, float eps, Workspace ws)
{
    constexpr int NCH = 2 * D;                  // q and k channels of one key head
    constexpr int EPC = 16 / (int)sizeof(Act);  // elements per 16-byte chunk
    constexpr int CPP = D / EPC;                // chunks per row of q (or k)
    constexpr int CPR = 2 * CPP;                // chunks per row of q | k
    constexpr int XR = kC + 3;                  // rows including the 3 halo rows
    constexpr int NCHUNK = XR * CPR;
    constexpr int LPT = (NCHUNK + 255) / 256;
    constexpr int XSC = CPR + 1;                // LDS row stride of raw x, in chunks
    constexpr int HS = D + 8;                   // fp16 row stride of q, k
    constexpr int AS = kC + 4;                  // fp32 row stride of A, Tinv
    constexpr int RS = 16 + 4;                  // fp32 row stride of a 16x16 staging tile
    constexpr int XBYTES = XR * XSC * 16;
    constexpr int ABYTES = 2 * kC * AS * 4;
    __shared__ __attribute__((aligned(16))) unsigned char ubuf[XBYTES > ABYTES ? XBYTES : ABYTES];
    __shared__ __attribute__((aligned(16))) _Float16 q16[kC * HS];
    __shared__ __attribute__((aligned(16))) _Float16 k16[kC * HS];
    __shared__ __attribute__((aligned(16))) float Rs[4][16 * RS];
    __shared__ float Gs[kC], bs[kC];
    u32x4 *const xs = (u32x4 *)ubuf;       // phases 1-2: raw x rows
    float *const As = (float *)ubuf;       // phase 4: A and Tinv
    float *const Ts = As + kC * AS;

    const int sub = blockIdx.x, kh = blockIdx.y;
    const int s = find_seg(sa, sub);
    const int64_t seg_row0 = sa.seg[s].row0;
    const int seg_n = sa.seg[s].n;
    const Act *win = (const Act *)sa.seg[s].win_in;
    const int r_base = (sub - sa.seg[s].sub0) * kC;
    const int nv = min(kC, seg_n - r_base);
    const int C = 2 * Hk * D + Hv * D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // 1. raw x rows r_base-3 .. r_base+63 of the q | k channels (16-byte loads, all in flight)
    {
        u32x4 buf[LPT];
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + 256 * i;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (idx < NCHUNK) {
                const int row = idx / CPR, cc = idx % CPR;
                const int ch = (cc / CPP) * Hk * D + kh * D + (cc % CPP) * EPC;
                const int sr = r_base + row - 3;
                if (sr < 0) {
                    if (conv_on) v = *(const u32x4 *)(win + (int64_t)(3 + sr) * C + ch);
                } else if (sr < seg_n) {
                    v = *(const u32x4 *)(x + (seg_row0 + sr) * C + ch);
                }
            }
            buf[i] = v;
        }
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + 256 * i;
            if (idx < NCHUNK) xs[(idx / CPR) * XSC + idx % CPR] = buf[i];
        }
    }
    __syncthreads();

    // 2. conv of 8 channels x RPT rows per thread, L2 norm reduced across the lanes of a row,
    //    normalised q, k as fp16 into LDS and the workspace
    {
        constexpr int G8 = NCH / 8, RP = 256 / G8, RPT = kC / RP;
        const int cg = tid % G8, rp = tid / G8;
        const int cl = cg * 8, part = cl / D, cd = cl % D;
        const int ch0 = part * Hk * D + kh * D + cd;
        float w[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int j = 0; j < 4; ++j) w[e][j] = conv_on ? to_f32(conv_w[(ch0 + e) * 4 + j]) : 0.f;
        _Float16 *dstl = part ? k16 : q16;
        _Float16 *dstg = (part ? ws.Kh : ws.Qh) + ((int64_t)sub * Hk + kh) * kC * D;
#pragma unroll
        for (int ri = 0; ri < RPT; ++ri) {
            const int r = rp * RPT + ri;
            float y[8];
            if (conv_on) {
                float xv[4][8];
#pragma unroll
                for (int j = 0; j < 4; ++j) load8<Act>(xs + (r + j) * XSC, cl, xv[j]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float a = w[e][0] * xv[0][e] + w[e][1] * xv[1][e] + w[e][2] * xv[2][e] +
                              w[e][3] * xv[3][e];
                    if (silu) a = a / (1.f + expf(-a));
                    y[e] = a;
                }
            } else {
                load8<Act>(xs + (r + 3) * XSC, cl, y);
            }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
#pragma unroll
            for (int off = 1; off < G8 / 2; off <<= 1) ss += __shfl_xor(ss, off);
            const float inv = (r < nv) ? 1.0f / sqrtf(ss + eps) : 0.f;
            half8 hv;
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = (_Float16)(y[e] * inv);
            *(half8 *)(dstl + r * HS + cd) = hv;
            *(half8 *)(dstg + r * D + cd) = hv;
        }
    }
    __syncthreads();

    // 3. K K^T and Q K^T, row tile `wave`, column tiles j <= wave
    f32x4 kk[4], qk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        qk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j <= wave) {
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) {
                const int off = 32 * kb + 8 * (lane / 16);
                const half8 ka = *(const half8 *)(k16 + (16 * wave + lane % 16) * HS + off);
                const half8 qa = *(const half8 *)(q16 + (16 * wave + lane % 16) * HS + off);
                const half8 kbv = *(const half8 *)(k16 + (16 * j + lane % 16) * HS + off);
                kk[j] = mfma16(ka, kbv, kk[j]);
                qk[j] = mfma16(qa, kbv, qk[j]);
            }
        }
    }

    // 4. per value head of this key head's group
    const int group = Hv / Hk;
    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        if (wave == 0) {  // cumulative log decay (inclusive scan) and beta; 0 past the end
            const int r = lane;
            float gv = (r < nv) ? g[(seg_row0 + r_base + r) * Hv + h] : 0.f;
            const float bv = (r < nv) ? beta[(seg_row0 + r_base + r) * Hv + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float t = __shfl_up(gv, off);
                if (lane >= off) gv += t;
            }
            Gs[r] = gv;
            bs[r] = bv;
            const float Gn = __shfl(gv, 63);
            const float gam = expf(gv);
            float *F = ws.Fac + ((int64_t)sub * Hv + h) * 4 * kC;
            F[r] = bv;
            F[kC + r] = bv * gam;
            F[2 * kC + r] = gam;
            F[3 * kC + r] = expf(Gn - gv);
        }
        __syncthreads();

        // A into LDS (fp32, zeros on and above the diagonal), M packed into the workspace
        {
            _Float16 *Mg = ws.Mm + ((int64_t)sub * Hv + h) * kPackedTri;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                half4 mv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * wave + 4 * (lane / 16) + i, c = 16 * j + lane % 16;
                    float a = 0.f, m = 0.f;
                    if (j <= wave && c <= r) {
                        const float dec = expf(Gs[r] - Gs[c]);
                        m = qk[j][i] * dec;
                        if (c < r) a = bs[r] * kk[j][i] * dec;
                    }
                    As[r * AS + c] = a;
                    mv[i] = (_Float16)m;
                }
                if (j <= wave) {
                    const int p = wave * (wave + 1) / 2 + j;
#pragma unroll
                    for (int i = 0; i < 4; ++i) Mg[p * 256 + i * 64 + lane] = mv[i];
                }
            }
        }
        __syncthreads();

        // Tinv = (I + A)^-1.  Phase 1: the four diagonal 16x16 blocks by forward substitution,
        // lane = 16 b + column (wave 0).  The other blocks of Ts are cleared meanwhile.
        if (wave == 0) {
            const int b = lane / 16, jj = lane % 16;
            float xv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == jj) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) acc -= As[(16 * b + r) * AS + 16 * b + i] * xv[i];
                xv[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Ts[(16 * b + r) * AS + 16 * b + jj] = xv[r];
        } else {
            for (int e = tid - 64; e < kC * kC; e += 192) {
                const int r = e / kC, c = e % kC;
                if ((r / 16) != (c / 16)) Ts[r * AS + c] = 0.f;
            }
        }
        __syncthreads();
        // Phase 2: row blocks b = 1..3; wave j < b makes tile (b, j):
        //   rhs = -A[b, j..b-1] Tinv[j..b-1, j];  Tinv[b, j] = Tinv[b, b] rhs   (fp32 MFMA)
        for (int b = 1; b < 4; ++b) {
            if (wave < b) {
                const int j = wave;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 16 * j; k0 < 16 * b; k0 += 4) {
                    const float a = As[(16 * b + lane % 16) * AS + k0 + lane / 16];
                    const float t = Ts[(k0 + lane / 16) * AS + 16 * j + lane % 16];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, t, acc, 0, 0, 0);
                }
                float *R = Rs[wave];
#pragma unroll
                for (int i = 0; i < 4; ++i) R[(4 * (lane / 16) + i) * RS + lane % 16] = -acc[i];
                f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4) {
                    const float a = Ts[(16 * b + lane % 16) * AS + 16 * b + k0 + lane / 16];
                    const float r = R[(k0 + lane / 16) * RS + lane % 16];
                    out = __builtin_amdgcn_mfma_f32_16x16x4f32(a, r, out, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Ts[(16 * b + 4 * (lane / 16) + i) * AS + 16 * j + lane % 16] = out[i];
            }
            __syncthreads();
        }
        // Tinv packed into the workspace (fp16)
        {
            _Float16 *Tg = ws.Tm + ((int64_t)sub * Hv + h) * kPackedTri;
            for (int idx = tid; idx < 10 * 32; idx += 256) {
                const int p = idx / 32, q = idx % 32;
                const float *src = Ts + (16 * tile_i(p) + chunk_row(q)) * AS + 16 * tile_j(p) + chunk_col(q);
                half8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = (_Float16)src[e];
                *(half8 *)(Tg + p * 256 + q * 8) = hv;
            }
        }
        __syncthreads();
    }
}

// One sub-chunk's chain inputs as staged in a loader thread's registers: K, Q, packed Tinv and
// M, raw v rows of this workgroup's 16 columns (with the 3 halo rows), and the factor table.
constexpr int kLoaders = 512;  // loader threads of a chain workgroup (waves 4..11)

template <int D, typename Act>
struct LoadSet {
    static constexpr int QKP = kC * D / 8 / kLoaders;  // 16-byte chunks of K (and Q) per thread
    static constexpr int TMC = 10 * 32;                // chunks of packed Tinv (and of M)
    static constexpr int TMP = (TMC + kLoaders - 1) / kLoaders;
    static constexpr int EPC = 16 / (int)sizeof(Act);
    static constexpr int VCR = 16 / EPC;               // chunks per v row (16 values)
    static constexpr int VC = (kC + 3) * VCR;
    static constexpr int VP = (VC + kLoaders - 1) / kLoaders;
    u32x4 k[QKP], q[QKP], t[TMP], m[TMP], v[VP], f;
};

struct ChainArgs {
    int sub0, seg_n, kh, h, Hk, Hv, C, vch, conv_on, c0;
    int64_t seg_row0;
};

// Loader side: issue the global loads of sub-chunk `cl` into `ls`.
template <int D, typename Act>
__device__ __forceinline__ void load_issue(LoadSet<D, Act> &ls, const ChainArgs &a, int lt, int cl,
                                           const Act *__restrict__ x, const Act *win,
                                           const Workspace &ws)
{
    using L = LoadSet<D, Act>;
    const int sub = a.sub0 + cl, rb = cl * kC;
    const u32x4 *Kg = (const u32x4 *)(ws.Kh + ((int64_t)sub * a.Hk + a.kh) * kC * D);
    const u32x4 *Qg = (const u32x4 *)(ws.Qh + ((int64_t)sub * a.Hk + a.kh) * kC * D);
#pragma unroll
    for (int i = 0; i < L::QKP; ++i) {
        ls.k[i] = Kg[lt + kLoaders * i];
        ls.q[i] = Qg[lt + kLoaders * i];
    }
    const u32x4 *Tg = (const u32x4 *)(ws.Tm + ((int64_t)sub * a.Hv + a.h) * kPackedTri);
    const u32x4 *Mg = (const u32x4 *)(ws.Mm + ((int64_t)sub * a.Hv + a.h) * kPackedTri);
#pragma unroll
    for (int i = 0; i < L::TMP; ++i) {
        const int idx = lt + kLoaders * i;
        ls.t[i] = u32x4{0u, 0u, 0u, 0u};
        ls.m[i] = u32x4{0u, 0u, 0u, 0u};
        if (idx < L::TMC) {
            ls.t[i] = Tg[idx];
            ls.m[i] = Mg[idx];
        }
    }
#pragma unroll
    for (int i = 0; i < L::VP; ++i) {
        const int idx = lt + kLoaders * i;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (idx < L::VC) {
            const int row = idx / L::VCR, cc = (idx % L::VCR) * L::EPC;
            const int sr = rb + row - 3;
            if (sr < 0) {
                if (a.conv_on) v = *(const u32x4 *)(win + (int64_t)(3 + sr) * a.C + a.vch + cc);
            } else if (sr < a.seg_n) {
                v = *(const u32x4 *)(x + (a.seg_row0 + sr) * a.C + a.vch + cc);
            }
        }
        ls.v[i] = v;
    }
    ls.f = u32x4{0u, 0u, 0u, 0u};
    if (lt < 64) ls.f = ((const u32x4 *)(ws.Fac + ((int64_t)sub * a.Hv + a.h) * 4 * kC))[lt];
}

// LDS of the chain kernel.  K, M and the factor table are double-buffered (read after the
// second barrier of a step while the next step's copy is written); Q, Tinv and the v rows are
// single (their last reader precedes the barrier after which the loader overwrites them).
template <int D, typename Act, typename Out>
struct ChainLds {
    static constexpr int HS = D + 8, TS = kC + 8, ST = D + 8;
    _Float16 k16[2][kC * HS];
    _Float16 q16[kC * HS];
    _Float16 t16[kC * TS];
    _Float16 m16[2][kC * TS];
    _Float16 s16t[16 * ST];
    _Float16 rt[16 * TS], dt[16 * TS], ddt[16 * TS];
    float fac[2][4 * kC];
    u32x4 xvr[LoadSet<D, Act>::VC];
    Out obuf[kC * 16];
};

template <int D, typename Act, typename Out>
__device__ __forceinline__ void load_put_early(ChainLds<D, Act, Out> &L, const LoadSet<D, Act> &ls,
                                               int lt, int buf)
{
    using LS = LoadSet<D, Act>;
    constexpr int HS = ChainLds<D, Act, Out>::HS, TS = ChainLds<D, Act, Out>::TS;
#pragma unroll
    for (int i = 0; i < LS::QKP; ++i) {
        const int idx = lt + kLoaders * i, r = idx / (D / 8), cc = (idx % (D / 8)) * 8;
        *(u32x4 *)(L.k16[buf] + r * HS + cc) = ls.k[i];
        *(u32x4 *)(L.q16 + r * HS + cc) = ls.q[i];
    }
#pragma unroll
    for (int i = 0; i < LS::TMP; ++i) {
        const int idx = lt + kLoaders * i;
        if (idx < LS::TMC) {
            const int p = idx / 32, q = idx % 32;
            *(u32x4 *)(L.m16[buf] + (16 * tile_i(p) + chunk_row(q)) * TS + 16 * tile_j(p) +
                       chunk_col(q)) = ls.m[i];
        }
    }
#pragma unroll
    for (int i = 0; i < LS::VP; ++i) {
        const int idx = lt + kLoaders * i;
        if (idx < LS::VC) L.xvr[idx] = ls.v[i];
    }
    if (lt < 64) ((u32x4 *)L.fac[buf])[lt] = ls.f;
}

template <int D, typename Act, typename Out>
__device__ __forceinline__ void load_put_t(ChainLds<D, Act, Out> &L, const LoadSet<D, Act> &ls, int lt)
{
    using LS = LoadSet<D, Act>;
    constexpr int TS = ChainLds<D, Act, Out>::TS;
#pragma unroll
    for (int i = 0; i < LS::TMP; ++i) {
        const int idx = lt + kLoaders * i;
        if (idx < LS::TMC) {
            const int p = idx / 32, q = idx % 32;
            *(u32x4 *)(L.t16 + (16 * tile_i(p) + chunk_row(q)) * TS + 16 * tile_j(p) + chunk_col(q)) =
                ls.t[i];
        }
    }
}

// Loader side: write the o tile of sub-chunk `cl` (staged in LDS by the compute waves).
template <int D, typename Act, typename Out>
__device__ __forceinline__ void store_o(const ChainLds<D, Act, Out> &L, const ChainArgs &a, int lt,
                                        int cl, Out *__restrict__ o)
{
    constexpr int OEPC = 16 / (int)sizeof(Out);  // outputs per 16-byte chunk
    constexpr int OCR = 16 / OEPC;               // chunks per row
    const int rb = cl * kC, nv = min(kC, a.seg_n - rb);
    if (lt < kC * OCR) {
        const int row = lt / OCR, cc = (lt % OCR) * OEPC;
        const u32x4 v = *(const u32x4 *)(L.obuf + row * 16 + cc);
        if (row < nv) *(u32x4 *)(o + ((a.seg_row0 + rb + row) * a.Hv + a.h) * D + a.c0 + cc) = v;
    }
}

// One loader step: K is the step index modulo 4 (static, so the register sets stay registers).
template <int K, int D, typename Act, typename Out>
__device__ __forceinline__ void loader_step(ChainLds<D, Act, Out> &L, LoadSet<D, Act> (&sets)[4],
                                            const ChainArgs &a, int lt, int cl, int nsub,
                                            const Act *__restrict__ x, const Act *win,
                                            const Workspace &ws, Out *__restrict__ o)
{
    if (cl >= nsub) return;
    const int nxt = (cl + 1) & 1;
    if (cl + 3 < nsub) load_issue<D, Act>(sets[(K + 3) % 4], a, lt, cl + 3, x, win, ws);
    if (cl > 0) store_o<D, Act, Out>(L, a, lt, cl - 1, o);
    __syncthreads();  // #1
    if (cl + 1 < nsub) load_put_early<D, Act, Out>(L, sets[(K + 1) % 4], lt, nxt);
    __syncthreads();  // #2
    if (cl + 1 < nsub) load_put_t<D, Act, Out>(L, sets[(K + 1) % 4], lt);
    __syncthreads();  // #3
}

// ------------------------------------------------------------------------------------------
// chain_kernel: the serial walk of one (d_v tile, value head, sequence) over its sub-chunks.
// Waves 0-3 compute; waves 4-11 load: they keep the inputs of the next three sub-chunks in
// flight in registers, write the next sub-chunk's inputs into LDS between the step's barriers
// and store each finished o tile, so the compute waves issue no global memory operation in
// the loop.  Every step has three barriers on both sides.
// ------------------------------------------------------------------------------------------
template <int D, typename Act, typename Out>
__global__ __launch_bounds__(256 + kLoaders) void chain_kernel(SegArgs sa, const Act *__restrict__ x,
                                                    const Act *__restrict__ conv_w, int conv_on,
                                                    int silu, int Hk, int Hv, float scale,
                                                    Workspace ws, Out *__restrict__ o)
{
    using CL = ChainLds<D, Act, Out>;
    constexpr int HS = CL::HS, TS = CL::TS, ST = CL::ST;
    constexpr int NT = D / 16;      // d_k tiles of the state
    constexpr int TPW = NT / 4;     // d_k tiles per compute wave
    __shared__ __attribute__((aligned(16))) CL L;

    // Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Units (value head,
    // tile) are numbered head-major, and XCD x takes a contiguous range of them, so the
    // workgroups that read one key head's K, Q (and one value head's factors) share an L2.
    const int NTILE = D / kTileV, n_units = Hv * NTILE, id = blockIdx.x;
    const int unit = (n_units % 8 == 0) ? (id % 8) * (n_units / 8) + id / 8 : id;
    const int tile = unit % NTILE, h = unit / NTILE, s = blockIdx.y;
    ChainArgs a;
    a.seg_row0 = sa.seg[s].row0;
    a.seg_n = sa.seg[s].n;
    a.sub0 = sa.seg[s].sub0;
    a.kh = h / (Hv / Hk);
    a.h = h;
    a.Hk = Hk;
    a.Hv = Hv;
    a.C = 2 * Hk * D + Hv * D;
    a.c0 = tile * 16;
    a.vch = 2 * Hk * D + h * D + a.c0;
    a.conv_on = conv_on;
    const Act *win = (const Act *)sa.seg[s].win_in;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nsub = (a.seg_n + kC - 1) / kC;

    if (wave >= 4) {
        // ---------------------------------------------------------------- loader waves
        const int lt = tid - 256;
        for (int e = lt; e < kC * kC; e += kLoaders) {  // tiles above the diagonal: zero, never written
            const int r = e / kC, c = e % kC;
            if (c / 16 > r / 16) {
                L.t16[r * TS + c] = (_Float16)0.f;
                L.m16[0][r * TS + c] = (_Float16)0.f;
                L.m16[1][r * TS + c] = (_Float16)0.f;
            }
        }
        LoadSet<D, Act> sets[4];
        if (nsub > 0) load_issue<D, Act>(sets[0], a, lt, 0, x, win, ws);
        if (nsub > 1) load_issue<D, Act>(sets[1], a, lt, 1, x, win, ws);
        if (nsub > 2) load_issue<D, Act>(sets[2], a, lt, 2, x, win, ws);
        if (nsub > 0) {
            load_put_early<D, Act, Out>(L, sets[0], lt, 0);
            load_put_t<D, Act, Out>(L, sets[0], lt);
        }
        __syncthreads();  // #0
        for (int cl = 0; cl < nsub; cl += 4) {
            loader_step<0>(L, sets, a, lt, cl, nsub, x, win, ws, o);
            loader_step<1>(L, sets, a, lt, cl + 1, nsub, x, win, ws, o);
            loader_step<2>(L, sets, a, lt, cl + 2, nsub, x, win, ws, o);
            loader_step<3>(L, sets, a, lt, cl + 3, nsub, x, win, ws, o);
        }
        if (nsub > 0) store_o<D, Act, Out>(L, a, lt, nsub - 1, o);
        return;
    }

    // -------------------------------------------------------------------- compute waves
    const int col = lane % 16, kg = lane / 16;
    const float *S_in = sa.seg[s].S_in;
    float *S_out = sa.seg[s].S_out;
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 1.f;
    if (conv_on) {
        w0 = to_f32(conv_w[(a.vch + col) * 4 + 0]);
        w1 = to_f32(conv_w[(a.vch + col) * 4 + 1]);
        w2 = to_f32(conv_w[(a.vch + col) * 4 + 2]);
        w3 = to_f32(conv_w[(a.vch + col) * 4 + 3]);
    }
    f32x4 S[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int kt = wave * TPW + t;
        half4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 16 * kt + 4 * kg + i;
            S[t][i] = S_in[((int64_t)h * D + k) * D + a.c0 + col];
            sv[i] = (_Float16)S[t][i];
        }
        *(half4 *)(L.s16t + col * ST + 16 * kt + 4 * kg) = sv;
    }
    __syncthreads();  // #0
    const Act *vrows = (const Act *)L.xvr;  // raw v of (halo ++ rows), 16 columns per row
    const int r0 = 16 * wave + 4 * kg;      // this lane's first row in the sub-chunk

    for (int cl = 0; cl < nsub; ++cl) {
        const int cur = cl & 1;
        const float *F = L.fac[cur];

        // X = K S and P = Q S for row tile `wave`
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) {
            const int off = 32 * kb + 8 * kg;
            const half8 bS = *(const half8 *)(L.s16t + col * ST + off);
            X = mfma16(*(const half8 *)(L.k16[cur] + (16 * wave + col) * HS + off), bS, X);
            P = mfma16(*(const half8 *)(L.q16 + (16 * wave + col) * HS + off), bS, P);
        }
        // R = beta V - beta gamma X; the state part of O is gamma P
        f32x4 Ob;
        {
            float vr[7];
#pragma unroll
            for (int j = 0; j < 7; ++j) vr[j] = to_f32(vrows[(r0 + j) * 16 + col]);
            half4 rv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + i;
                float v = w0 * vr[i] + w1 * vr[i + 1] + w2 * vr[i + 2] + w3 * vr[i + 3];
                if (silu && conv_on) v = v / (1.f + expf(-v));
                rv[i] = (_Float16)(F[r] * v - F[kC + r] * X[i]);
                Ob[i] = F[2 * kC + r] * P[i];
            }
            *(half4 *)(L.rt + col * TS + r0) = rv;
        }
        __syncthreads();  // #1

        // D = Tinv R (tiles above the diagonal of Tinv are zero)
        f32x4 Dl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int off = 32 * kb + 8 * kg;
            Dl = mfma16(*(const half8 *)(L.t16 + (16 * wave + col) * TS + off),
                        *(const half8 *)(L.rt + col * TS + off), Dl);
        }
        {
            half4 dv, ddv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dv[i] = (_Float16)Dl[i];
                ddv[i] = (_Float16)(F[3 * kC + r0 + i] * Dl[i]);
            }
            *(half4 *)(L.dt + col * TS + r0) = dv;
            *(half4 *)(L.ddt + col * TS + r0) = ddv;
        }
        __syncthreads();  // #2

        // S' = gamma_n S + K^T (exp(G_n - G) D)
        {
            const float gn = F[2 * kC + kC - 1];
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int kt = wave * TPW + t;
                f32x4 acc = S[t] * gn;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int off = 32 * kb + 8 * kg;
                    acc = mfma16(ktrans_frag(L.k16[cur], HS, 32 * kb, 16 * kt, lane),
                                 *(const half8 *)(L.ddt + col * TS + off), acc);
                }
                S[t] = acc;
                half4 sv;
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[i] = (_Float16)acc[i];
                *(half4 *)(L.s16t + col * ST + 16 * kt + 4 * kg) = sv;
            }
        }
        // O = scale (gamma Q S + M D), staged in LDS for the loader waves
        {
            f32x4 Oa = Ob;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int off = 32 * kb + 8 * kg;
                Oa = mfma16(*(const half8 *)(L.m16[cur] + (16 * wave + col) * TS + off),
                            *(const half8 *)(L.dt + col * TS + off), Oa);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) store_out(L.obuf + (r0 + i) * 16 + col, scale * Oa[i]);
        }
        __syncthreads();  // #3
    }

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int kt = wave * TPW + t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 16 * kt + 4 * kg + i;
            S_out[((int64_t)h * D + k) * D + a.c0 + col] = S[t][i];
        }
    }
}

// ------------------------------------------------------------------------------------------
// window_kernel: window_out = rows n .. n+2 of (window_in ++ x), bit copies, per channel
// ------------------------------------------------------------------------------------------
template <typename Act>
__global__ __launch_bounds__(256) void window_kernel(SegArgs sa, const Act *__restrict__ x, int C)
{
    const int s = blockIdx.y;
    const int ch = blockIdx.x * 256 + threadIdx.x;
    if (ch >= C) return;
    const Act *wi = (const Act *)sa.seg[s].win_in;
    Act *wo = (Act *)sa.seg[s].win_out;
    const int64_t n = sa.seg[s].n, row0 = sa.seg[s].row0;
    Act v[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int64_t r = n + i;
        v[i] = (r < 3) ? wi[r * C + ch] : x[(row0 + r - 3) * C + ch];
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) wo[(int64_t)i * C + ch] = v[i];
}

// ------------------------------------------------------------------------------------------
// conv_step_kernel: standalone causal conv over all channels (window read, not written)
// ------------------------------------------------------------------------------------------
template <typename Act, typename Out>
__global__ __launch_bounds__(256) void conv_step_kernel(const Act *__restrict__ x,
                                                        const Act *__restrict__ w,
                                                        const Act *__restrict__ win,
                                                        Out *__restrict__ y, int64_t T, int C,
                                                        int silu, int rows_per_block)
{
    const int ch = blockIdx.x * 256 + threadIdx.x;
    if (ch >= C) return;
    const int64_t ra = (int64_t)blockIdx.y * rows_per_block;
    const int64_t rb = min(T, ra + rows_per_block);
    auto xt = [&](int64_t r) -> float {
        return r < 0 ? to_f32(win[(3 + r) * C + ch]) : to_f32(x[r * C + ch]);
    };
    const float w0 = to_f32(w[ch * 4 + 0]), w1 = to_f32(w[ch * 4 + 1]);
    const float w2 = to_f32(w[ch * 4 + 2]), w3 = to_f32(w[ch * 4 + 3]);
    float a0 = xt(ra - 3), a1 = xt(ra - 2), a2 = xt(ra - 1);
    for (int64_t r = ra; r < rb; ++r) {
        const float a3 = xt(r);
        float v = w0 * a0 + w1 * a1 + w2 * a2 + w3 * a3;
        if (silu) v = v / (1.f + expf(-v));
        store_out(y + r * C + ch, v);
        a0 = a1;
        a1 = a2;
        a2 = a3;
    }
}

__global__ void zero_kernel(uint32_t *p, size_t n_words)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ void copy_kernel(uint32_t *dst, const uint32_t *src, size_t n_words)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
struct EventMarks {
    void *const *ev;
    int n;
    hipStream_t st;
    void mark(int i) const
    {
        if (ev && i < n && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], st);
    }
};

template <int D, typename Act, typename Out>
static int prefill_t(const gdn_desc &d, const SegArgs &sa, const void *x, const void *conv_w,
                     const float *g, const float *beta, void *o, const Workspace &ws,
                     hipStream_t st, const EventMarks &em)
{
    const int conv_on = d.conv_width > 0 ? 1 : 0;
    const int C = 2 * d.n_k_heads * D + d.n_v_heads * D;
    em.mark(0);
    hipLaunchKernelGGL((prep_kernel<D, Act>), dim3(sa.n_sub, d.n_k_heads), dim3(256), 0, st, sa,
                       (const Act *)x, (const Act *)conv_w, conv_on, d.conv_silu, g, beta,
                       d.n_k_heads, d.n_v_heads, d.l2_eps, ws);
    em.mark(1);
    em.mark(2);
    hipLaunchKernelGGL((chain_kernel<D, Act, Out>), dim3((D / kTileV) * d.n_v_heads, sa.n_seg),
                       dim3(256 + kLoaders), 0, st, sa, (const Act *)x, (const Act *)conv_w, conv_on,
                       d.conv_silu, d.n_k_heads, d.n_v_heads, d.scale, ws, (Out *)o);
    em.mark(3);
    em.mark(4);
    if (conv_on)
        hipLaunchKernelGGL((window_kernel<Act>), dim3((C + 255) / 256, sa.n_seg), dim3(256), 0, st,
                           sa, (const Act *)x, C);
    em.mark(5);
    return (int)hipGetLastError();
}

template <int D>
static int prefill_d(const gdn_desc &d, const SegArgs &sa, const void *x, const void *conv_w,
                     const float *g, const float *beta, void *o, const Workspace &ws,
                     hipStream_t st, const EventMarks &em)
{
    if (d.act_dtype == GDN_BF16) {
        if (d.out_dtype == GDN_BF16)
            return prefill_t<D, bf16_t, bf16_t>(d, sa, x, conv_w, g, beta, o, ws, st, em);
        return prefill_t<D, bf16_t, float>(d, sa, x, conv_w, g, beta, o, ws, st, em);
    }
    if (d.out_dtype == GDN_BF16)
        return prefill_t<D, float, bf16_t>(d, sa, x, conv_w, g, beta, o, ws, st, em);
    return prefill_t<D, float, float>(d, sa, x, conv_w, g, beta, o, ws, st, em);
}

int launch_prefill(const gdn_desc &d, const SegArgs &sa, const void *x, const void *conv_w,
                   const float *g, const float *beta, void *o, const Workspace &ws, void *stream,
                   void *const *events, int n_events)
{
    (void)hipGetLastError();  // clear a stale error so the check below reports ours
    hipStream_t st = (hipStream_t)stream;
    const EventMarks em{events, n_events, st};
    if (d.d_k == 128) return prefill_d<128>(d, sa, x, conv_w, g, beta, o, ws, st, em);
    return prefill_d<64>(d, sa, x, conv_w, g, beta, o, ws, st, em);
}

template <typename Act, typename Out>
static int conv_t(const gdn_desc &d, const void *x, const void *w, void *window, void *y,
                  int64_t T, hipStream_t st)
{
    const int C = 2 * d.n_k_heads * d.d_k + d.n_v_heads * d.d_v;
    const int rpb = 64;
    const int64_t nb = (T + rpb - 1) / rpb;
    if (T > 0) {
        hipLaunchKernelGGL((conv_step_kernel<Act, Out>), dim3((C + 255) / 256, (unsigned)nb),
                           dim3(256), 0, st, (const Act *)x, (const Act *)w, (const Act *)window,
                           (Out *)y, T, C, d.conv_silu, rpb);
        // the window becomes rows T .. T+2 of (window ++ x); in place, per channel
        SegArgs sa;
        memset(&sa, 0, sizeof(sa));
        sa.n_seg = 1;
        sa.seg[0].row0 = 0;
        sa.seg[0].n = (int32_t)T;
        sa.seg[0].win_in = window;
        sa.seg[0].win_out = window;
        hipLaunchKernelGGL((window_kernel<Act>), dim3((C + 255) / 256, 1), dim3(256), 0, st, sa,
                           (const Act *)x, C);
    }
    return (int)hipGetLastError();
}

int launch_conv_step(const gdn_desc &d, const void *x, const void *conv_w, void *window, void *y,
                     int64_t T, void *stream)
{
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)stream;
    if (d.act_dtype == GDN_BF16) {
        if (d.out_dtype == GDN_BF16) return conv_t<bf16_t, bf16_t>(d, x, conv_w, window, y, T, st);
        return conv_t<bf16_t, float>(d, x, conv_w, window, y, T, st);
    }
    if (d.out_dtype == GDN_BF16) return conv_t<float, bf16_t>(d, x, conv_w, window, y, T, st);
    return conv_t<float, float>(d, x, conv_w, window, y, T, st);
}

int launch_zero(void *p, size_t bytes, void *stream)
{
    if (bytes == 0) return 0;
    (void)hipGetLastError();
    const size_t words = bytes / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (uint32_t *)p, words);
    return (int)hipGetLastError();
}

int launch_copy(void *dst, const void *src, size_t bytes, void *stream)
{
    if (bytes == 0) return 0;
    (void)hipGetLastError();
    const size_t words = bytes / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (uint32_t *)dst, (const uint32_t *)src, words);
    return (int)hipGetLastError();
}

}  // namespace gdn
