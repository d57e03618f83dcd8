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
//   prep_kernel    one workgroup per (sub-chunk, key head), key head fastest: conv of the
//                  q|k channels, L2 norm, K K^T and Q K^T on MFMA, and for each value head of
//                  the group the cumulative gates, Tinv (blocked forward substitution in LDS,
//                  fp32) and the decayed mask M.
//                  Everything it writes is independent of the state, so all sub-chunks run
//                  in parallel.
//   chain_kernel   grid (d_v tiles of 16, value heads, sequences), 8 waves: the serial walk
//                  over the sub-chunks.  Columns of S evolve independently, so each workgroup
//                  owns S[:, 16 columns] in MFMA accumulators (fp32) for the whole call, with an
//                  fp16 copy in LDS as the MFMA operand.  Four waves run the recurrence, four
//                  compute the outputs, convolve the workgroup's v columns and stage the shared
//                  tables.  It also writes the sequence's new conv window.
//   window_kernel  the new conv window = the last 3 rows of (window ++ x), copied bit for bit
//                  (the standalone conv step).
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
    return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
}
__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t *p, float v) { p->bits = f32_to_bf16_bits(v); }

// Store four adjacent output elements starting at element offset `off` (a multiple of 4) of a
// raw buffer; dropped when out of range.
template <typename Out>
__device__ __forceinline__ void store_out4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v);
template <>
__device__ __forceinline__ void store_out4<float>(__amdgpu_buffer_rsrc_t r, int off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off * 4, 0, 0);
}
template <>
__device__ __forceinline__ void store_out4<bf16_t>(__amdgpu_buffer_rsrc_t r, int off, f32x4 v)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = {(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                     (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off * 2, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c)
{
    // D[m][n] += sum_k A[m][k] B[k][n], 16x16x32.  Lane l supplies A[l%16][8(l/16) .. +7] and
    // B[8(l/16) .. +7][l%16]; it receives D[4(l/16) + i][l%16], i = 0..3.
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef short short4_t __attribute__((ext_vector_type(4)));

// Half offset of K[t][c] in a K tile: the 16-byte chunk c / 8 of row t is XORed with a
// permutation of the low four bits of t.  The 16 rows that a 16-lane group writes then hit
// distinct chunks, and so do the 8 rows x 2 chunks that 32 lanes of a transposed read
// (ds_read_b64_tr_b16) touch: both are free of bank conflicts.
__device__ __forceinline__ int k_off(int t, int c)
{
    const int f = ((t >> 3) & 1) * 8 + ((t >> 1) & 1) * 4 + (t & 1) * 2 + ((t >> 2) & 1);
    return t * 128 + 8 * ((c >> 3) ^ f) + (c & 7);
}

// Half offset of element p of row `col` in a [16][128] tile (S^T, R^T, D^T): the 8-byte chunk
// p / 4 is XORed with 2 col.  A 16-byte B-fragment read (chunks 2m, 2m+1) stays contiguous,
// and the 16 columns read by a lane group hit distinct chunk pairs.
__device__ __forceinline__ int c_off(int col, int p) { return col * 128 + 4 * ((p >> 2) ^ (2 * col)) + (p & 3); }

// A fragment of K^T for the 16x16x32 MFMA read straight from the K tile in LDS (k_off):
// lane (m, kg) of the result holds K[r0 + 8 kg + e][c0 + m], e = 0..7.  ds_read_b64_tr_b16
// hands lane i of each 16-lane group element i % 4 of the 4-element reads of lanes
// 4 e + i / 4, so lane j reads K[row0 + j / 4][c0 + 4 (j % 4) .. + 3] (rows row0 .. row0 + 3).
__device__ __forceinline__ half8 ktrans_frag(const _Float16 *K, int r0, int c0, int lane)
{
    const int j = lane % 16, kg = lane / 16;
    const int r = r0 + 8 * kg + j / 4, c = c0 + 4 * (j % 4);
    typedef __attribute__((address_space(3))) short4_t lds_short4;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(K + k_off(r, c)));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(K + k_off(r + 4, c)));
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

// Fragment (w, kb) of a lower-triangular factor: its index among the stored ones, or -1 when
// every column of the K step lies above the diagonal of row tile w (the fragment is zero).
__device__ __forceinline__ int tri_frag(int w, int kb) { return kb == 0 ? (w < 2 ? w : 2 * w - 2) : (w < 2 ? -1 : 2 * w - 1); }

constexpr int cmax(int a, int b) { return a > b ? a : b; }

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

// Sum over aligned groups of N lanes (N = 8 or 16), the result in every lane of the group:
// a butterfly of DPP moves (quad permutations, then the half-row and row mirrors).
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
#define GDN_DPP_ADD(ctrl) \
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xf, 0xf, false))
    GDN_DPP_ADD(0xb1);   // quad_perm [1, 0, 3, 2]
    GDN_DPP_ADD(0x4e);   // quad_perm [2, 3, 0, 1]
    GDN_DPP_ADD(0x141);  // row_half_mirror
    if constexpr (N == 16) GDN_DPP_ADD(0x140);  // row_mirror
#undef GDN_DPP_ADD
    return v;
}

// ------------------------------------------------------------------------------------------
// prep_kernel: state-independent factors of one (sub-chunk, key head).
// ------------------------------------------------------------------------------------------
template <int D, typename Act, bool SILU>
__global__ __launch_bounds__(256, 3) void prep_kernel(SegArgs sa, const Act *__restrict__ x,
                                                      const Act *__restrict__ conv_w, int conv_on,
                                                      const float *__restrict__ g,
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
    constexpr int XBYTES = XR * XSC * 16;
    constexpr int QBYTES = kC * HS * 2;
    // A and Tinv of a value head are kept as their ten lower 16x16 blocks (b, j), j <= b,
    // block index b (b + 1) / 2 + j, rows of 20 floats, blocks 324 floats apart (the four
    // diagonal blocks then start in different LDS banks).
    constexpr int BROW = 20, BSTR = 16 * BROW + 4;
    constexpr int MBYTES = 10 * BSTR * 4;
    constexpr int UBYTES = cmax(cmax(XBYTES, 2 * QBYTES), 4 * MBYTES);
    // Phase 1 keeps the raw x rows, phases 2-3 q16 and k16 over the same bytes, phase 4 A and
    // Tinv of two value heads over them again.
    __shared__ __attribute__((aligned(16))) unsigned char ubuf[UBYTES];
    __shared__ __attribute__((aligned(16))) float Gs[2][kC], bs[2][kC];
    u32x4 *const xs = (u32x4 *)ubuf;
    _Float16 *const q16 = (_Float16 *)ubuf;
    _Float16 *const k16 = q16 + kC * HS;
#define AS_OF(hh) ((float *)(ubuf + (hh) * MBYTES))
#define TS_OF(hh) ((float *)(ubuf + (2 + (hh)) * MBYTES))
#define BLK(b, j) (((b) * ((b) + 1) / 2 + (j)) * BSTR)

    // units are numbered key head fastest, so the workgroups that run together read whole rows
    // of x (every key head's q | k channels of the same sub-chunk) rather than one column slice
    // of many sub-chunks
    const int sub = blockIdx.x / Hk, kh = blockIdx.x % Hk;
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
        float w[8][4];  // taps of channels ch0 .. ch0+7: 32 consecutive values of conv_w
        {
            u32x4 wc[8 * (int)sizeof(Act) / 4];
#pragma unroll
            for (int q = 0; q < 8 * (int)sizeof(Act) / 4; ++q)
                wc[q] = conv_on ? ((const u32x4 *)(conv_w + ch0 * 4))[q] : u32x4{0u, 0u, 0u, 0u};
            const Act *wv = (const Act *)wc;
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j) w[e][j] = to_f32(wv[e * 4 + j]);
        }
        _Float16 *dstl = part ? k16 : q16;
        // rows rp*RPT .. +RPT-1; the conv reads raw rows r .. r+3, kept as a rolling window
        float xw[4][8];
        half8 outv[RPT];
        if (conv_on) {
#pragma unroll
            for (int j = 0; j < 3; ++j) load8<Act>(xs + (rp * RPT + j) * XSC, cl, xw[j + 1]);
        }
#pragma unroll
        for (int ri = 0; ri < RPT; ++ri) {
            const int r = rp * RPT + ri;
            float y[8];
            if (conv_on) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xw[0][e] = xw[1][e];
                    xw[1][e] = xw[2][e];
                    xw[2][e] = xw[3][e];
                }
                load8<Act>(xs + (r + 3) * XSC, cl, xw[3]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float a = w[e][0] * xw[0][e] + w[e][1] * xw[1][e] + w[e][2] * xw[2][e] +
                              w[e][3] * xw[3][e];
                    if constexpr (SILU) a = a / (1.f + __expf(-a));
                    y[e] = a;
                }
            } else {
                load8<Act>(xs + (r + 3) * XSC, cl, y);
            }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
            ss = group_sum<G8 / 2>(ss);
            const float inv = (r < nv) ? __builtin_amdgcn_rsqf(ss + eps) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) outv[ri][e] = (_Float16)(y[e] * inv);
        }
        __syncthreads();  // raw rows no longer read; q16 and k16 take their bytes
#pragma unroll
        for (int ri = 0; ri < RPT; ++ri) *(half8 *)(dstl + (rp * RPT + ri) * HS + cd) = outv[ri];
    }
    __syncthreads();

    // normalised q, k to the workspace in MFMA A-fragment order (coalesced for the chain)
    {
        _Float16 *Qg = (_Float16 *)ws.Qh + ((int64_t)sub * Hk + kh) * kC * D;
        _Float16 *Kg = (_Float16 *)ws.Kh + ((int64_t)sub * Hk + kh) * kC * D;
        for (int c = tid; c < kC * D / 8; c += 256) {
            const int f = c / 64, l = c % 64, w = f / (D / 32), kb = f % (D / 32);
            const int off = (16 * w + l % 16) * HS + 32 * kb + 8 * (l / 16);
            *(half8 *)(Qg + c * 8) = *(const half8 *)(q16 + off);
            *(half8 *)(Kg + c * 8) = *(const half8 *)(k16 + off);
        }
    }

    // 3. K K^T and Q K^T for row tile `wave`, column tiles j <= wave, with the operands swapped
    //    so that lane (g = lane / 16, cc = lane % 16) holds, for column tile j, the entries
    //    [16 wave + cc][16 j + 4 g + i], i = 0..3: one row per lane, four adjacent columns.
    f32x4 kk[4], qk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        qk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j <= wave) {
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) {
                const int off = 32 * kb + 8 * (lane / 16);
                const half8 kw = *(const half8 *)(k16 + (16 * wave + lane % 16) * HS + off);
                const half8 qw = *(const half8 *)(q16 + (16 * wave + lane % 16) * HS + off);
                const half8 kj = *(const half8 *)(k16 + (16 * j + lane % 16) * HS + off);
                kk[j] = mfma16(kj, kw, kk[j]);
                qk[j] = mfma16(kj, qw, qk[j]);
            }
        }
    }

    // 4. the value heads of this key head's group, two at a time (head pair slot hh = 0, 1)
    const int group = Hv / Hk;
    const int g4 = lane / 16, cc = lane % 16;
    const int row = 16 * wave + cc;  // this lane's row of the Gram tiles
    for (int hp = 0; hp < group; hp += 2) {
        const int nh = min(2, group - hp);
        if (wave < nh) {  // cumulative log decay (inclusive scan) and beta; 0 past the end
            const int h = kh * group + hp + wave, r = lane;
            float gv = (r < nv) ? g[(seg_row0 + r_base + r) * Hv + h] : 0.f;
            const float bv = (r < nv) ? beta[(seg_row0 + r_base + r) * Hv + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float t = __shfl_up(gv, off);
                if (lane >= off) gv += t;
            }
            Gs[wave][r] = gv;
            bs[wave][r] = bv;
            const float Gn = __shfl(gv, 63);
            const float gam = __expf(gv);
            float *F = ws.Fac + ((int64_t)sub * Hv + h) * 4 * kC;
            F[r] = bv;
            F[kC + r] = bv * gam;
            F[2 * kC + r] = gam;
            F[3 * kC + r] = __expf(Gn - gv);
        }
        __syncthreads();  // gates ready; raw rows, q16 and k16 are no longer read

        // A = strict_lower(beta K K^T * decay) into LDS (fp32); M = lower(Q K^T * decay) from
        // registers to the workspace.  Fragment (w, kb) of M, lane l, element e holds column
        // 32 kb + 16 (e / 4) + 4 (l / 16) + e % 4 of row 16 w + l % 16, which is this lane's
        // tile 2 kb + e / 4, entry e % 4.
        for (int hh = 0; hh < nh; ++hh) {
            const int h = kh * group + hp + hh;
            const float Gr = Gs[hh][row], br = bs[hh][row];
            f32x4 mt[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (j <= wave) {
                    const f32x4 Gc = *(const f32x4 *)(&Gs[hh][16 * j + 4 * g4]);
                    f32x4 at;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = 16 * j + 4 * g4 + i;
                        const float dec = (c <= row) ? __expf(Gr - Gc[i]) : 0.f;
                        mt[j][i] = qk[j][i] * dec;
                        at[i] = (c < row) ? br * kk[j][i] * dec : 0.f;
                    }
                    *(f32x4 *)(AS_OF(hh) + BLK(wave, j) + cc * BROW + 4 * g4) = at;
                }
            }
            _Float16 *Mg = (_Float16 *)ws.Mm + ((int64_t)sub * Hv + h) * kPackedTri;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb == 0 || wave >= 2) {
                    half8 hv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) hv[e] = (_Float16)mt[2 * kb + e / 4][e % 4];
                    *(half8 *)(Mg + (tri_frag(wave, kb) * 64 + lane) * 8) = hv;
                }
            }
        }
        __syncthreads();  // A complete

        // Tinv = (I + A)^-1 by 16 x 16 blocks.  Diagonal blocks by forward substitution
        // (wave hh, lane = 16 b + column).
        // The strictly lower rows of the block are read as 16-byte pieces, four rows at a
        // time and all before their use, so that the reads overlap one another instead of each
        // waiting for the last; a row's sum is accumulated in order over its columns.
        if (wave < nh) {
            const float *Ab = AS_OF(wave) + BLK(lane / 16, lane / 16);
            float *Th = TS_OF(wave);
            const int b = lane / 16, jj = lane % 16;
            float xv[16];
#pragma unroll
            for (int part = 0; part < 4; ++part) {
                f32x4 ar[4][4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 4 * part + rr;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (4 * q < r) ar[rr][q] = *(const f32x4 *)(Ab + r * BROW + 4 * q);
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 4 * part + rr;
                    float acc = (r == jj) ? 1.f : 0.f;
#pragma unroll
                    for (int i = 0; i < r; ++i) acc -= ar[rr][i / 4][i % 4] * xv[i];
                    xv[r] = acc;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Th[BLK(b, b) + r * BROW + jj] = xv[r];
        }
        __syncthreads();  // diagonal blocks complete

        // Tinv[b1][b0] = -Tinv[b1][b1] (A[b1][b0] Tinv[b0][b0]) for (b1, b0) = (1, 0), (3, 2):
        // wave = 2 hh + p takes p = 0, 1 of head slot hh.
        const int hw = wave / 2, pw = wave % 2;
        if (hw < nh) {
            const float *Ah = AS_OF(hw);
            float *Th = TS_OF(hw);
            const int b0 = 2 * pw, b1 = b0 + 1;
            f32x4 rhs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const float av = Ah[BLK(b1, b0) + cc * BROW + 4 * s4 + g4];
                const float bv = Th[BLK(b0, b0) + (4 * s4 + g4) * BROW + cc];
                rhs = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, rhs, 0, 0, 0);
            }
            // rhs as the B operand: step s supplies k = 4 g + s, i.e. this lane's entry s
            f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const float av = Th[BLK(b1, b1) + cc * BROW + 4 * g4 + s4];
                out = __builtin_amdgcn_mfma_f32_16x16x4f32(av, rhs[s4], out, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) Th[BLK(b1, b0) + (4 * g4 + i) * BROW + cc] = -out[i];
        }
        __syncthreads();  // blocks (1,0) and (3,2) complete

        // Lower-left 32 x 32 block: W_i = sum_{l = jc..1} A[i][l] Tinv[l][jc] (i = 2, 3), then
        // Tinv[2][jc] = -Tinv[2][2] W_2, Tinv[3][jc] = -(Tinv[3][2] W_2 + Tinv[3][3] W_3).
        // wave = 2 hh + jc.
        if (hw < nh) {
            const float *Ah = AS_OF(hw);
            float *Th = TS_OF(hw);
            const int jc = pw;
            f32x4 W2 = {0.f, 0.f, 0.f, 0.f}, W3 = {0.f, 0.f, 0.f, 0.f};
            for (int l = jc; l < 2; ++l) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const float tv = Th[BLK(l, jc) + (4 * s4 + g4) * BROW + cc];
                    const float a2 = Ah[BLK(2, l) + cc * BROW + 4 * s4 + g4];
                    const float a3 = Ah[BLK(3, l) + cc * BROW + 4 * s4 + g4];
                    W2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, tv, W2, 0, 0, 0);
                    W3 = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, tv, W3, 0, 0, 0);
                }
            }
            f32x4 T2 = {0.f, 0.f, 0.f, 0.f}, T3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int kc = 4 * g4 + s4;
                T2 = __builtin_amdgcn_mfma_f32_16x16x4f32(Th[BLK(2, 2) + cc * BROW + kc], W2[s4], T2, 0, 0, 0);
                T3 = __builtin_amdgcn_mfma_f32_16x16x4f32(Th[BLK(3, 2) + cc * BROW + kc], W2[s4], T3, 0, 0, 0);
                T3 = __builtin_amdgcn_mfma_f32_16x16x4f32(Th[BLK(3, 3) + cc * BROW + kc], W3[s4], T3, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Th[BLK(2, jc) + (4 * g4 + i) * BROW + cc] = -T2[i];
                Th[BLK(3, jc) + (4 * g4 + i) * BROW + cc] = -T3[i];
            }
        }
        __syncthreads();  // Tinv complete

        // Tinv to the workspace as fragments, with the column order of the M fragments
        for (int c = tid; c < nh * kTriFrags * 64; c += 256) {
            const int hh = c / (kTriFrags * 64), f = (c / 64) % kTriFrags, l = c % 64;
            const int w = f < 2 ? f : 2 + (f - 2) / 2, kb = f < 2 ? 0 : (f - 2) % 2;
            const float *Th = TS_OF(hh);
            const int off = (l % 16) * BROW + 4 * (l / 16);
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};  // blocks above the diagonal
            const f32x4 lo = (2 * kb <= w) ? *(const f32x4 *)(Th + BLK(w, 2 * kb) + off) : z4;
            const f32x4 hi = (2 * kb + 1 <= w) ? *(const f32x4 *)(Th + BLK(w, 2 * kb + 1) + off) : z4;
            half8 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hv[e] = (_Float16)lo[e];
                hv[4 + e] = (_Float16)hi[e];
            }
            const int h = kh * group + hp + hh;
            *(half8 *)((_Float16 *)ws.Tm + ((int64_t)sub * Hv + h) * kPackedTri + (f * 64 + l) * 8) = hv;
        }
        if (hp + 2 < group) __syncthreads();  // A, Tinv and the gates are reused by the next pair
    }
#undef AS_OF
#undef TS_OF
#undef BLK
}

// ------------------------------------------------------------------------------------------
// chain_kernel: the serial walk of one (d_v tile, value head, sequence) over its sub-chunks.
//
// Eight waves, two per SIMD, in two roles that meet at the same three barriers per step:
//   state waves 0-3  the recurrence.  Wave c computes rows 16c .. 16c+15 of X = K S and of
//                    D = Tinv R, and d_k rows 32c .. 32c+31 (D = 128) of the state tile, which
//                    it keeps in fp32 registers for the whole call.
//   output waves 4-7 everything off the recurrence: P = Q S, O = scale (gamma P + M D) and
//                    its store, and beta * conv(v) of the next sub-chunk.
// Every wave loads the fragments and gate factors it uses straight into its own registers,
// two sub-chunks ahead; LDS carries what one wave computes for another (S^T, R^T, D^T,
// beta conv(v)), K for its transposed reads, and the raw v rows of the conv.  The LDS unit
// and the vector-memory queue are the scarce resources of a step, so:
//  - every LDS tile is laid out so that its reads and writes are free of bank conflicts
//    (rows of 256 bytes whose 8- or 16-byte chunks are XOR-swizzled by row; see k_off and
//    c_off), which halves the cycles the unit spends per instruction;
//  - the raw v rows come in with one 16-byte load per output thread and pass through LDS, not
//    as seven 2-byte loads per lane;
//  - the three phases are balanced in LDS instructions:
//   phase 1  state: X = K S (S from LDS), R = beta v - beta gamma X -> LDS
//            output: O of the previous sub-chunk (its D still in LDS), stored; the raw v
//                   rows and factors of the next sub-chunk -> LDS
//   phase 2  state: D = Tinv R -> LDS (as is, and times exp(G_n - G)); K rows of the next
//                   sub-chunk -> LDS
//            output: P = Q S (S read here rather than in phase 1), times gamma
//   phase 3  state: S' = gamma_n S + K^T (exp(G_n - G) D); its fp16 copy -> LDS
//            output: beta * conv(v) of the next sub-chunk -> LDS
// ------------------------------------------------------------------------------------------

// What a state wave loads for one sub-chunk: its K (A operand of X) and Tinv (A operand of D)
// fragments.
template <int D>
struct StateRegs {
    static constexpr int KB = D / 32;  // 32-wide K steps over d_k
    half8 kf[KB], tf[2];
};

// What an output wave loads for one sub-chunk: Q and M fragments, and LP 16-byte chunks bound
// for LDS: the raw v rows of this workgroup's 16 columns (3 halo rows + 64), then the 1 KB
// factor table (every wave reads factors of many rows, so one copy in LDS serves all).
template <int D, typename Act>
struct OutRegs {
    static constexpr int KB = D / 32;
    static constexpr int EPC = 16 / (int)sizeof(Act);
    static constexpr int VCR = 16 / EPC;               // chunks per v row (16 values)
    static constexpr int VC = (kC + 3) * VCR;          // v chunks
    // In LDS each raw v row takes one chunk more than its 16 values: the conv's 2- or 4-byte
    // reads of rows 4 apart then fall in different banks (without the pad they meet two ways).
    static constexpr int VRS = VCR + 1;
    static constexpr int NLD = VC + 64;                // + factor table chunks
    static constexpr int LP = (NLD + 255) / 256;       // chunks per output thread
    half8 qf[KB], mf[2];
    u32x4 ld[LP];
};

struct ChainArgs {
    int sub0, seg_n, kh, h, Hk, Hv, C, vch, c0, wave, col, kg, ot;
    int64_t seg_row0;
    // Buffer resources: their range checks return 0 for reads outside the sequence (rows past
    // its end or before its start) and drop writes outside it, so loads and stores need no
    // branches.
    __amdgpu_buffer_rsrc_t rx;  // x rows of the sequence, from its first row
    __amdgpu_buffer_rsrc_t ro;  // o rows of the sequence
};

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// State-wave prefetch of sub-chunk `cl`: PART 1 the K fragments, 2 the Tinv fragments.
template <int D, int PART>
__device__ __forceinline__ void state_issue(StateRegs<D> &R, const ChainArgs &a, int cl,
                                            const Workspace &ws)
{
    using SR = StateRegs<D>;
    const int sub = a.sub0 + cl;
    const int lane = 16 * a.kg + a.col;
    if constexpr (PART == 1) {
        const half8 *Kg = (const half8 *)(ws.Kh + ((int64_t)sub * a.Hk + a.kh) * kC * D) + a.wave * SR::KB * 64 + lane;
#pragma unroll
        for (int kb = 0; kb < SR::KB; ++kb) R.kf[kb] = Kg[kb * 64];
    } else {
        const half8 *Tg = (const half8 *)(ws.Tm + ((int64_t)sub * a.Hv + a.h) * kPackedTri) + lane;
        R.tf[0] = Tg[64 * tri_frag(a.wave, 0)];
        R.tf[1] = (a.wave >= 2) ? Tg[64 * tri_frag(a.wave, 1)] : half8{};  // wave-uniform
    }
}

// Output-wave prefetch of sub-chunk `cl`: PART 1 the Q fragments, 2 the M fragments, 3 the raw
// v rows and the factor table.
template <int D, typename Act, int PART>
__device__ __forceinline__ void out_issue(OutRegs<D, Act> &R, const ChainArgs &a, int cl,
                                          const Workspace &ws)
{
    using OR = OutRegs<D, Act>;
    const int sub = a.sub0 + cl;
    const int lane = 16 * a.kg + a.col;
    if constexpr (PART == 1) {
        const half8 *Qg = (const half8 *)(ws.Qh + ((int64_t)sub * a.Hk + a.kh) * kC * D) + a.wave * OR::KB * 64 + lane;
#pragma unroll
        for (int kb = 0; kb < OR::KB; ++kb) R.qf[kb] = Qg[kb * 64];
    } else if constexpr (PART == 2) {
        const half8 *Mg = (const half8 *)(ws.Mm + ((int64_t)sub * a.Hv + a.h) * kPackedTri) + lane;
        R.mf[0] = Mg[64 * tri_frag(a.wave, 0)];
        R.mf[1] = (a.wave >= 2) ? Mg[64 * tri_frag(a.wave, 1)] : half8{};  // wave-uniform
    } else {
        const u32x4 *Fg = (const u32x4 *)(ws.Fac + ((int64_t)sub * a.Hv + a.h) * 4 * kC);
#pragma unroll
        for (int i = 0; i < OR::LP; ++i) {
            const int idx = a.ot + 256 * i;
            if (idx < OR::VC) {
                const int vr = idx / OR::VCR, cc = (idx % OR::VCR) * OR::EPC;
                const int sr = cl * kC + vr - 3;  // sequence-local row (rows before 0: the window, added apart)
                R.ld[i] = __builtin_amdgcn_raw_buffer_load_b128(a.rx, (sr * a.C + a.vch + cc) * (int)sizeof(Act), 0, 0);
            } else {
                R.ld[i] = Fg[min(idx - OR::VC, 63)];
            }
        }
    }
}

// LDS of the chain kernel.  Every fp16 tile has rows of 128 halves (256 bytes, all 64 banks).
template <int D, typename Act>
struct ChainLds {
    static constexpr int RW = 128, BS = kC + 8;
    _Float16 k16[2][kC * RW];              // K rows of this step (transposed reads), double-buffered
    _Float16 s16t[16 * RW];                // S^T, fp16: the B operand of X and P
    _Float16 rt[16 * RW], dt[16 * RW], ddt[16 * RW];  // R^T, D^T, (exp(G_n - G) D)^T
    float bv[16 * BS];                     // beta * conv(v) of the next step, [column][row]
    u32x4 xvr[(kC + 3) * OutRegs<D, Act>::VRS];  // raw v rows of the next step (3 halo rows + 64)
    float fac[2][4 * kC];                  // per row: beta, beta*gamma, gamma, exp(G_n - G)
};


// Output wave: the raw v rows and the factor table of register set R into LDS (factor buffer
// `buf`).  The halo rows of a sequence's first sub-chunk come from the conv window (`win`
// non-null): the x loads returned 0 there.
template <int D, typename Act>
__device__ __forceinline__ void put_ld(ChainLds<D, Act> &L, const OutRegs<D, Act> &R, const ChainArgs &a,
                                       int buf, const Act *win)
{
    using OR = OutRegs<D, Act>;
#pragma unroll
    for (int i = 0; i < OR::LP; ++i) {
        const int idx = a.ot + 256 * i;
        u32x4 v = R.ld[i];
        if (idx < OR::VC) {
            const int vr = idx / OR::VCR, ci = idx % OR::VCR;
            if (win != nullptr && idx < 3 * OR::VCR)
                v = v | *(const u32x4 *)(win + (int64_t)vr * a.C + a.vch + ci * OR::EPC);
            L.xvr[vr * OR::VRS + ci] = v;
        } else if (idx < OR::NLD) {
            ((u32x4 *)L.fac[buf])[idx - OR::VC] = v;
        }
    }
}

// Output wave: beta * conv(v) of rows 16 wave + 4 kg .. +3, column col, from the raw rows in
// LDS and beta of factor buffer `buf`, into L.bv.
template <int D, typename Act, bool SILU>
__device__ __forceinline__ void conv_bv(ChainLds<D, Act> &L, const ChainArgs &a, int buf, float w0,
                                        float w1, float w2, float w3)
{
    using CL = ChainLds<D, Act>;
    const int r0 = 16 * a.wave + 4 * a.kg;
    constexpr int RS = OutRegs<D, Act>::VRS * OutRegs<D, Act>::EPC;  // row stride, in values
    const Act *vrows = (const Act *)L.xvr;
    float vr[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) vr[j] = to_f32(vrows[(r0 + j) * RS + a.col]);
    const f32x4 fb = *(const f32x4 *)(L.fac[buf] + r0);
    f32x4 bvv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = w0 * vr[i] + w1 * vr[i + 1] + w2 * vr[i + 2] + w3 * vr[i + 3];
        if constexpr (SILU) v = v / (1.f + expf(-v));
        bvv[i] = fb[i] * v;
    }
    *(f32x4 *)(L.bv + a.col * CL::BS + r0) = bvv;
}

// One step of a state wave over sub-chunk `cl` with register set K (step index modulo NB, the
// depth of the prefetch ring: the loads of a sub-chunk go out NB - 1 steps before its own).
template <int K, int NB, int D, typename Act>
__device__ __forceinline__ void state_step(ChainLds<D, Act> &L, StateRegs<D> (&R)[NB], const ChainArgs &a,
                                           int cl, int nsub, f32x4 (&S)[D / 64], const Workspace &ws)
{
    using CL = ChainLds<D, Act>;
    using SR = StateRegs<D>;
    constexpr int TPW = D / 64;  // d_k tiles per wave
    const StateRegs<D> &C = R[K];
    const int wave = a.wave, col = a.col, kg = a.kg, lane = a.kg * 16 + a.col;
    const int r0 = 16 * wave + 4 * kg;
    // Tinv and M fragments order their 32-wide K steps as (4 rows of tile 2kb, 4 rows of tile
    // 2kb+1) per lane group; rt and dt hold the rows of R and D in that order, so that their
    // B fragments stay 16 contiguous bytes: row 16w + 4kg + i sits at position pr0 + i.
    const int pr0 = 32 * (wave / 2) + 8 * kg + 4 * (wave % 2);
    const float *F = L.fac[cl & 1];
    const int cn = min(cl + NB - 1, nsub - 1);  // the sub-chunk whose inputs this step prefetches
    state_issue<D, 1>(R[(K + NB - 1) % NB], a, cn, ws);

    // phase 1: X = K S for row tile `wave`; R = beta v - beta gamma X
    f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < SR::KB; ++kb)
        X = mfma16(C.kf[kb], *(const half8 *)(L.s16t + c_off(col, 32 * kb + 8 * kg)), X);
    {
        const f32x4 bv = *(const f32x4 *)(L.bv + col * CL::BS + r0);
        const f32x4 fbg = *(const f32x4 *)(F + kC + r0);
        half4 rv;
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[i] = (_Float16)(bv[i] - fbg[i] * X[i]);
        *(half4 *)(L.rt + c_off(col, pr0)) = rv;
    }
    __syncthreads();  // #1: rt complete

    // phase 2: D = Tinv R (fragments above the diagonal are zero); this step's K rows for the
    // transposed reads of phase 3
    state_issue<D, 2>(R[(K + NB - 1) % NB], a, cn, ws);
    f32x4 Dl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        Dl = mfma16(C.tf[kb], *(const half8 *)(L.rt + c_off(col, 32 * kb + 8 * kg)), Dl);
    {
        _Float16 *kn = L.k16[cl & 1];
#pragma unroll
        for (int kb = 0; kb < SR::KB; ++kb)
            *(half8 *)(kn + k_off(16 * wave + col, 32 * kb + 8 * kg)) = C.kf[kb];
    }
    {
        const f32x4 fd = *(const f32x4 *)(F + 3 * kC + r0);
        half4 dv, ddv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dv[i] = (_Float16)Dl[i];
            ddv[i] = (_Float16)(fd[i] * Dl[i]);
        }
        *(half4 *)(L.dt + c_off(col, pr0)) = dv;
        *(half4 *)(L.ddt + c_off(col, r0)) = ddv;
    }
    __syncthreads();  // #2: dt, ddt and the K rows complete

    // phase 3: S' = gamma_n S + K^T (exp(G_n - G) D)
    {
        const _Float16 *kc = L.k16[cl & 1];
        half8 bd[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) bd[kb] = *(const half8 *)(L.ddt + c_off(col, 32 * kb + 8 * kg));
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int kt = wave * TPW + t;
            f32x4 acc = S[t] * F[3 * kC - 1];  // gamma_n: gamma of the last row
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                acc = mfma16(ktrans_frag(kc, 32 * kb, 16 * kt, lane), bd[kb], acc);
            S[t] = acc;
            half4 sv;
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = (_Float16)acc[i];
            *(half4 *)(L.s16t + c_off(col, 16 * kt + 4 * kg)) = sv;
        }
    }
    __syncthreads();  // #3: s16t complete for the next step
}

// Output wave: O of sub-chunk `cl` = scale (gamma P + M D), transposed (D^T M^T) like P, from
// Ob = gamma P, the M fragments mf and D^T in LDS; this lane stores row 16 wave + col,
// columns 4 kg .. +3.
template <int D, typename Act, typename Out>
__device__ __forceinline__ void out_store(const ChainLds<D, Act> &L, const ChainArgs &a, int cl, f32x4 Ob,
                                          const half8 (&mf)[2], float scale)
{
    f32x4 Oa = Ob;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        Oa = mfma16(*(const half8 *)(L.dt + c_off(a.col, 32 * kb + 8 * a.kg)), mf[kb], Oa);
    const int obase = ((cl * kC + 16 * a.wave + a.col) * a.Hv + a.h) * D + a.c0 + 4 * a.kg;
    store_out4<Out>(a.ro, obase, Oa * scale);
}

// One step of an output wave over sub-chunk `cl` with register set K (of NB).  Ob and mcur carry
// gamma P and the M fragments of the previous sub-chunk into this step's phase 1.  Q and M are
// loaded NB - 1 steps ahead; the raw v rows, which come from HBM, NB steps ahead: set K then
// takes those of sub-chunk cl + NB (its previous rows, of sub-chunk cl, went to LDS one step
// ago).
template <int K, int NB, int D, typename Act, typename Out, bool SILU>
__device__ __forceinline__ void out_step(ChainLds<D, Act> &L, OutRegs<D, Act> (&R)[NB], const ChainArgs &a,
                                         int cl, int nsub, f32x4 &Ob, half8 (&mcur)[2], float w0,
                                         float w1, float w2, float w3, float scale,
                                         const Workspace &ws)
{
    using OR = OutRegs<D, Act>;
    const OutRegs<D, Act> &C = R[K];
    const int col = a.col, kg = a.kg;
    const int cn = min(cl + NB - 1, nsub - 1);

    // phase 1: O of the previous sub-chunk (its D^T is in LDS until this step's phase 2); the
    // next sub-chunk's raw v rows and factors
    if (cl > 0) out_store<D, Act, Out>(L, a, cl - 1, Ob, mcur, scale);
    put_ld<D, Act>(L, R[(K + 1) % NB], a, (cl + 1) & 1, nullptr);
    out_issue<D, Act, 3>(R[K], a, min(cl + NB, nsub - 1), ws);
    __syncthreads();  // #1

    // phase 2: P = Q S, transposed (D^T of S^T Q^T): this lane's row 16 wave + col, columns
    // 4 kg .. +3; the state part of O is gamma P
    f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < OR::KB; ++kb)
        P = mfma16(*(const half8 *)(L.s16t + c_off(col, 32 * kb + 8 * kg)), C.qf[kb], P);
    Ob = P * L.fac[cl & 1][2 * kC + 16 * a.wave + col];
    mcur[0] = C.mf[0];
    mcur[1] = C.mf[1];
    out_issue<D, Act, 2>(R[(K + NB - 1) % NB], a, cn, ws);
    __syncthreads();  // #2: dt complete

    // phase 3: beta * conv(v) of the next step
    if (cl + 1 < nsub) conv_bv<D, Act, SILU>(L, a, (cl + 1) & 1, w0, w1, w2, w3);
    out_issue<D, Act, 1>(R[(K + NB - 1) % NB], a, cn, ws);
    __syncthreads();  // #3: bv complete for the next step
}

// NB 3 fits one workgroup per CU (158 VGPRs at D = 128); NB 2 keeps every wave within 128 VGPRs
// so that two workgroups share a CU, for launches with at least two workgroups per CU.
template <int D, typename Act, typename Out, bool SILU, int NB>
__global__ __launch_bounds__(512, NB == 2 ? 4 : 2) void chain_kernel(SegArgs sa, const Act *__restrict__ x,
                                                    const Act *__restrict__ conv_w, int conv_on,
                                                    int Hk, int Hv, float scale, Workspace ws,
                                                    Out *__restrict__ o)
{
    using CL = ChainLds<D, Act>;
    constexpr int TPW = D / 64;
    __shared__ __attribute__((aligned(16))) CL L;

    // Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Units (value head,
    // tile) are numbered head-major, and XCD x takes a contiguous range of them, so the
    // workgroups that read one key head's K, Q (and one value head's factors) share an L2.
    const int NTILE = D / kTileV, n_units = Hv * NTILE, id = blockIdx.x;
    const int unit = (n_units % 8 == 0) ? (id % 8) * (n_units / 8) + id / 8 : id;
    const int tile = unit % NTILE, h = unit / NTILE, s = blockIdx.y;
    const bool state_role = threadIdx.x < 256;  // waves 0-3; waves 4-7 are output waves
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
    a.ot = threadIdx.x & 255;
    a.wave = (threadIdx.x >> 6) & 3;
    a.col = threadIdx.x % 16;
    a.kg = (threadIdx.x & 63) / 16;
    const Act *win = (const Act *)sa.seg[s].win_in;
    const float *S_in = sa.seg[s].S_in;
    float *S_out = sa.seg[s].S_out;
    const int nsub = (a.seg_n + kC - 1) / kC;
    const int wave = a.wave, col = a.col, kg = a.kg;
    a.rx = __builtin_amdgcn_make_buffer_rsrc((void *)(x + a.seg_row0 * a.C), 0,
                                             a.seg_n * a.C * (int)sizeof(Act), kRsrcWord3);
    a.ro = __builtin_amdgcn_make_buffer_rsrc((void *)(o + a.seg_row0 * Hv * D), 0,
                                             a.seg_n * Hv * D * (int)sizeof(Out), kRsrcWord3);

    if (state_role) {
        StateRegs<D> R[NB];
        if (nsub > 0) {
            state_issue<D, 1>(R[0], a, 0, ws);
            state_issue<D, 2>(R[0], a, 0, ws);
            if constexpr (NB == 3) {
                state_issue<D, 1>(R[1], a, min(1, nsub - 1), ws);
                state_issue<D, 2>(R[1], a, min(1, nsub - 1), ws);
            }
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
            *(half4 *)(L.s16t + c_off(col, 16 * kt + 4 * kg)) = sv;
        }
        __syncthreads();  // prologue #1
        __syncthreads();  // prologue #2
        // Whole rounds of NB steps first, with no exits inside: every load issued in the loop is
        // then consumed on every path, and the compiler's waits stay behind the loads.
        int cl = 0;
        for (; cl + NB <= nsub; cl += NB) {
            state_step<0, NB, D, Act>(L, R, a, cl, nsub, S, ws);
            state_step<1, NB, D, Act>(L, R, a, cl + 1, nsub, S, ws);
            if constexpr (NB == 3) state_step<2, NB, D, Act>(L, R, a, cl + 2, nsub, S, ws);
        }
        if (cl < nsub) state_step<0, NB, D, Act>(L, R, a, cl, nsub, S, ws);
        if constexpr (NB == 3)
            if (cl + 1 < nsub) state_step<1, NB, D, Act>(L, R, a, cl + 1, nsub, S, ws);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int kt = wave * TPW + t;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 16 * kt + 4 * kg + i;
                S_out[((int64_t)h * D + k) * D + a.c0 + col] = S[t][i];
            }
        }
    } else {
        float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 1.f;
        if (conv_on) {
            w0 = to_f32(conv_w[(a.vch + col) * 4 + 0]);
            w1 = to_f32(conv_w[(a.vch + col) * 4 + 1]);
            w2 = to_f32(conv_w[(a.vch + col) * 4 + 2]);
            w3 = to_f32(conv_w[(a.vch + col) * 4 + 3]);
        }
        OutRegs<D, Act> R[NB];
        f32x4 Ob = {0.f, 0.f, 0.f, 0.f};
        half8 mcur[2] = {half8{}, half8{}};
        if (nsub > 0) {
            out_issue<D, Act, 3>(R[0], a, 0, ws);
            out_issue<D, Act, 3>(R[1], a, min(1, nsub - 1), ws);
            if constexpr (NB == 3) out_issue<D, Act, 3>(R[2], a, min(2, nsub - 1), ws);
            out_issue<D, Act, 1>(R[0], a, 0, ws);
            out_issue<D, Act, 2>(R[0], a, 0, ws);
            if constexpr (NB == 3) {
                out_issue<D, Act, 1>(R[1], a, min(1, nsub - 1), ws);
                out_issue<D, Act, 2>(R[1], a, min(1, nsub - 1), ws);
            }
            put_ld<D, Act>(L, R[0], a, 0, conv_on ? win : nullptr);
        }
        __syncthreads();  // prologue #1: raw v rows and factors of step 0 in LDS
        if (nsub > 0) conv_bv<D, Act, SILU>(L, a, 0, w0, w1, w2, w3);
        __syncthreads();  // prologue #2: bv of step 0 in LDS
        int cl = 0;
        for (; cl + NB <= nsub; cl += NB) {
            out_step<0, NB, D, Act, Out, SILU>(L, R, a, cl, nsub, Ob, mcur, w0, w1, w2, w3, scale, ws);
            out_step<1, NB, D, Act, Out, SILU>(L, R, a, cl + 1, nsub, Ob, mcur, w0, w1, w2, w3, scale, ws);
            if constexpr (NB == 3)
                out_step<2, NB, D, Act, Out, SILU>(L, R, a, cl + 2, nsub, Ob, mcur, w0, w1, w2, w3, scale, ws);
        }
        if (cl < nsub) out_step<0, NB, D, Act, Out, SILU>(L, R, a, cl, nsub, Ob, mcur, w0, w1, w2, w3, scale, ws);
        if constexpr (NB == 3)
            if (cl + 1 < nsub)
                out_step<1, NB, D, Act, Out, SILU>(L, R, a, cl + 1, nsub, Ob, mcur, w0, w1, w2, w3, scale, ws);
        // O of the last sub-chunk: its D^T was completed at the last step's barrier #2
        if (nsub > 0) out_store<D, Act, Out>(L, a, nsub - 1, Ob, mcur, scale);
    }

    // The new conv window: rows n .. n+2 of (window ++ x), per channel.  This workgroup
    // rewrites the 16 v channels whose old window it read above, and one slice of the q | k
    // channels (whose old window only the prep kernel read, before this kernel started).  Each
    // thread takes one channel and reads its three values before writing them back.
    Act *win_out = (Act *)sa.seg[s].win_out;
    if (conv_on && win_out != nullptr) {
        const int nqk = 2 * Hk * D, per = (nqk + n_units - 1) / n_units;
        const int t = threadIdx.x;
        int ch = -1;
        if (t < 16) ch = a.vch + t;
        else if (t < 16 + per && unit * per + (t - 16) < nqk) ch = unit * per + (t - 16);
        if (ch >= 0) {
            Act v[3];
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int64_t r = (int64_t)a.seg_n + i;
                v[i] = (r < 3) ? win[r * a.C + ch] : x[(a.seg_row0 + r - 3) * a.C + ch];
            }
#pragma unroll
            for (int i = 0; i < 3; ++i) win_out[(int64_t)i * a.C + ch] = v[i];
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
// conv_step_kernel: standalone causal conv over all channels (window read, not written).
// Thread t of the grid's x extent takes 8 adjacent channels (one 16-byte load of bf16, two of
// fp32) over one block of rows, keeping the last three inputs of each channel in registers; a
// wave reads and writes 64 x 8 contiguous channels of a row per instruction.
// ------------------------------------------------------------------------------------------
template <typename Act>
__device__ __forceinline__ void load8_row(const Act *p, float (&v)[8])
{
    if constexpr (sizeof(Act) == 2) {
        const u32x4 u = *(const u32x4 *)p;
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[4 + e] = b[e];
        }
    }
}

template <typename Out>
__device__ __forceinline__ void store8_row(Out *p, const float (&v)[8])
{
    if constexpr (sizeof(Out) == 2) {
        u32x4 u;
        u.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        u.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        u.z = (uint32_t)f32_to_bf16_bits(v[4]) | ((uint32_t)f32_to_bf16_bits(v[5]) << 16);
        u.w = (uint32_t)f32_to_bf16_bits(v[6]) | ((uint32_t)f32_to_bf16_bits(v[7]) << 16);
        *(u32x4 *)p = u;
    } else {
        *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4 *)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

template <typename Act, typename Out>
__global__ __launch_bounds__(256) void conv_step_kernel(const Act *__restrict__ x,
                                                        const Act *__restrict__ w,
                                                        const Act *__restrict__ win,
                                                        Out *__restrict__ y, int64_t T, int C,
                                                        int silu, int rows_per_block)
{
    const int ch = 8 * (blockIdx.x * 256 + threadIdx.x);
    if (ch >= C) return;
    const int64_t ra = (int64_t)blockIdx.y * rows_per_block;
    const int64_t rb = min(T, ra + rows_per_block);
    float wt[8][4];  // taps of channels ch .. ch+7: 32 consecutive values of w
    {
        float t[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) load8_row<Act>(w + (int64_t)ch * 4 + 8 * q, *(float(*)[8])(t + 8 * q));
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int j = 0; j < 4; ++j) wt[e][j] = t[4 * e + j];
    }
    float a[3][8];  // inputs of rows r-3, r-2, r-1
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t r = ra - 3 + j;
        load8_row<Act>(r < 0 ? win + (3 + r) * C + ch : x + r * C + ch, a[j]);
    }
    for (int64_t r = ra; r < rb; ++r) {
        float cur[8], out[8];
        load8_row<Act>(x + r * C + ch, cur);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = wt[e][0] * a[0][e] + wt[e][1] * a[1][e] + wt[e][2] * a[2][e] + wt[e][3] * cur[e];
            if (silu) v = v / (1.f + expf(-v));
            out[e] = v;
            a[0][e] = a[1][e];
            a[1][e] = a[2][e];
            a[2][e] = cur[e];
        }
        store8_row<Out>(y + r * C + ch, out);
    }
}

// ------------------------------------------------------------------------------------------
// decode_kernel: one token of one sequence per grid row, one (value head, 32-column tile of S)
// per workgroup.  The per-token rule in fp32:
//   q, k, v = conv(window ++ x) of the token; q^ = q / sqrt(|q|^2 + eps), k^ likewise;
//   u = S^T k^;  e = v - e^g u;  S' = e^g S + beta k^ e^T;  o = scale S'^T q^
// (S' = e^g (I - beta k^ k^T) S + beta k^ v^T).  Thread (r, c) = (t / 8, t % 8) holds columns
// 4c .. 4c+3 of the tile at rows r, r + 32, ...: each of its loads and stores of S is 16 bytes,
// and a wave's covers 8 rows x 128 contiguous bytes.  The column sums u and o are reduced
// over the 8 row groups of a wave by lane swaps, then over the 4 waves through LDS, in a fixed
// order.  The new conv window (the last W-1 inputs) is written here only into a window other
// than the one read (several workgroups read the q | k window of a key head): the workgroup of
// tile 0 of a key head's first value head writes the q | k channels, every workgroup its own v
// channels.  For an in-place window, window_kernel shifts it afterwards.
// ------------------------------------------------------------------------------------------
template <int D, typename Act, typename Out, bool SILU>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs da, const Act *__restrict__ conv_w,
                                                     int conv_on, int Hk, int Hv, float scale,
                                                     float eps)
{
    constexpr int W = 32, NT = D / W, RPT = D / 32;
    constexpr int NQK = 2 * D / 8;  // threads converting 8 q | k channels each
    __shared__ float qk[2 * D];      // q | k of the key head after the conv (not yet normalised)
    __shared__ float ve[W];          // conv(v) of the tile, then e
    __shared__ float red[4][W];      // column partial sums of the 4 waves
    __shared__ float inv[2];         // 1 / sqrt(|q|^2 + eps), 1 / sqrt(|k|^2 + eps)
    const int h = blockIdx.x / NT, tile = blockIdx.x % NT, b = blockIdx.y;
    const DecodeSeq sq = da.seq[b];
    const int kh = h / (Hv / Hk), C = 2 * Hk * D + Hv * D;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const Act *x = (const Act *)sq.x, *win = (const Act *)sq.win;
    // this thread's part of the S tile, loaded first so that it is in flight during the conv
    const int r = t / 8, c4 = 4 * (t % 8);
    const f32x4 *Sin = (const f32x4 *)(sq.S_in + (int64_t)h * D * D + tile * W + c4);
    f32x4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) sv[i] = Sin[(int64_t)(r + 32 * i) * (D / 4)];
    // 1. conv: threads 0 .. NQK-1 take 8 q | k channels each, the next 4 threads 8 channels of
    //    the tile's v; 16-byte loads of the row, the window rows and the taps
    const int vt = t - NQK;
    if (t < NQK || (vt >= 0 && vt < 4)) {
        const int ch = t < NQK ? (8 * t < D ? 0 : Hk * D) + kh * D + (8 * t) % D
                               : 2 * Hk * D + h * D + tile * W + 8 * vt;
        float xr[8], w0r[8], w1r[8], w2r[8];
        load8<Act>((const u32x4 *)x, ch, xr);
        float y[8];
        if (conv_on) {
            load8<Act>((const u32x4 *)win, ch, w0r);
            load8<Act>((const u32x4 *)(win + C), ch, w1r);
            load8<Act>((const u32x4 *)(win + 2 * C), ch, w2r);
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // taps of channels ch + 2q, ch + 2q + 1
                float tp[8];
                load8<Act>((const u32x4 *)conv_w, 4 * ch + 8 * q, tp);
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    const int e = 2 * q + e2;
                    float a = tp[4 * e2] * w0r[e] + tp[4 * e2 + 1] * w1r[e] + tp[4 * e2 + 2] * w2r[e] +
                              tp[4 * e2 + 3] * xr[e];
                    if constexpr (SILU) a = a / (1.f + expf(-a));
                    y[e] = a;
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = xr[e];
        }
        float *dst = t < NQK ? qk + 8 * t : ve + 8 * vt;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = y[e];
        // the new window, when it is not the one read: the workgroup of tile 0 of a key
        // head's first value head writes the q | k channels, every workgroup its own v ones
        if (conv_on && sq.win_out != nullptr && (t >= NQK || (tile == 0 && h % (Hv / Hk) == 0))) {
            Act *wo = (Act *)sq.win_out;
            *(u32x4 *)(wo + ch) = *(const u32x4 *)(win + C + ch);
            *(u32x4 *)(wo + C + ch) = *(const u32x4 *)(win + 2 * C + ch);
            *(u32x4 *)(wo + 2 * C + ch) = *(const u32x4 *)(x + ch);
            if constexpr (sizeof(Act) == 4) {
                *(u32x4 *)(wo + ch + 4) = *(const u32x4 *)(win + C + ch + 4);
                *(u32x4 *)(wo + C + ch + 4) = *(const u32x4 *)(win + 2 * C + ch + 4);
                *(u32x4 *)(wo + 2 * C + ch + 4) = *(const u32x4 *)(x + ch + 4);
            }
        }
    }
    __syncthreads();
    // 2. L2 norms: wave 0 sums q^2, wave 1 k^2
    if (wave < 2) {
        float s2 = 0.f;
        for (int i = lane; i < D; i += 64) s2 += qk[wave * D + i] * qk[wave * D + i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s2 += __shfl_xor(s2, off);
        if (lane == 0) inv[wave] = 1.f / sqrtf(s2 + eps);
    }
    const float alpha = expf(sq.g[h]), bt = sq.beta[h];
    __syncthreads();
    const float iq = inv[0], ik = inv[1];
    // column sums of this thread's 4 columns over the wave's 8 row groups (lanes 8 apart),
    // then over the 4 waves
    auto colsum = [&](f32x4 p) {
#pragma unroll
        for (int off = 8; off < 64; off <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] += __shfl_xor(p[e], off);
        if (lane < 8) *(f32x4 *)&red[wave][c4] = p;
    };
    // 3. u = S^T k^, then e = v - e^g u
    f32x4 pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) pu += (qk[D + r + 32 * i] * ik) * sv[i];
    colsum(pu);
    __syncthreads();
    if (t < W) ve[t] = ve[t] - alpha * (((red[0][t] + red[1][t]) + red[2][t]) + red[3][t]);
    __syncthreads();
    // 4. S' = e^g S + beta k^ e^T, stored; o = scale S'^T q^
    const f32x4 ej = *(const f32x4 *)&ve[c4];
    f32x4 *Sout = (f32x4 *)(sq.S_out + (int64_t)h * D * D + tile * W + c4);
    f32x4 po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = r + 32 * i;
        const f32x4 sn = alpha * sv[i] + (bt * (qk[D + d] * ik)) * ej;
        Sout[(int64_t)d * (D / 4)] = sn;
        po += (qk[d] * iq) * sn;
    }
    colsum(po);  // red was last read before the barrier above
    __syncthreads();
    if (t < W) {
        const float ov = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
        store_out((Out *)sq.o + h * D + tile * W + t, ov * scale);
    }
}

template <int D, typename Act, typename Out>
static int decode_t(const gdn_desc &d, const DecodeArgs &da, const SegArgs &wa, const void *x,
                    const void *conv_w, hipStream_t st)
{
    const int conv_on = d.conv_width > 0 ? 1 : 0;
    const dim3 grid((D / 32) * d.n_v_heads, da.n);
    if (d.conv_silu && conv_on)
        hipLaunchKernelGGL((decode_kernel<D, Act, Out, true>), grid, dim3(256), 0, st, da,
                           (const Act *)conv_w, conv_on, d.n_k_heads, d.n_v_heads, d.scale, d.l2_eps);
    else
        hipLaunchKernelGGL((decode_kernel<D, Act, Out, false>), grid, dim3(256), 0, st, da,
                           (const Act *)conv_w, conv_on, d.n_k_heads, d.n_v_heads, d.scale, d.l2_eps);
    if (conv_on && wa.n_seg > 0) {
        const int C = 2 * d.n_k_heads * d.d_k + d.n_v_heads * d.d_v;
        hipLaunchKernelGGL((window_kernel<Act>), dim3((C + 255) / 256, wa.n_seg), dim3(256), 0, st,
                           wa, (const Act *)x, C);
    }
    return (int)hipGetLastError();
}

int launch_decode(const gdn_desc &d, const DecodeArgs &da, const SegArgs &wa, const void *x,
                  const void *conv_w, void *stream)
{
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)stream;
    if (d.d_k == 128) {
        if (d.act_dtype == GDN_BF16)
            return d.out_dtype == GDN_BF16 ? decode_t<128, bf16_t, bf16_t>(d, da, wa, x, conv_w, st)
                                           : decode_t<128, bf16_t, float>(d, da, wa, x, conv_w, st);
        return d.out_dtype == GDN_BF16 ? decode_t<128, float, bf16_t>(d, da, wa, x, conv_w, st)
                                       : decode_t<128, float, float>(d, da, wa, x, conv_w, st);
    }
    if (d.act_dtype == GDN_BF16)
        return d.out_dtype == GDN_BF16 ? decode_t<64, bf16_t, bf16_t>(d, da, wa, x, conv_w, st)
                                       : decode_t<64, bf16_t, float>(d, da, wa, x, conv_w, st);
    return d.out_dtype == GDN_BF16 ? decode_t<64, float, bf16_t>(d, da, wa, x, conv_w, st)
                                   : decode_t<64, float, float>(d, da, wa, x, conv_w, st);
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

// The chain kernel's ring depth for a launch of n_wg workgroups: 2 (two workgroups per CU) once
// there are at least two per CU, else 3.
static bool chain_ring2(int64_t n_wg)
{
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    return n_cu > 0 && n_wg >= 2 * (int64_t)n_cu;
}

template <int D, typename Act, typename Out>
static int prefill_t(const gdn_desc &d, const SegArgs &sa, const void *x, const void *conv_w,
                     const float *g, const float *beta, void *o, const Workspace &ws,
                     hipStream_t st, const EventMarks &em)
{
    const int conv_on = d.conv_width > 0 ? 1 : 0;
    em.mark(0);
    if (d.conv_silu && conv_on)
        hipLaunchKernelGGL((prep_kernel<D, Act, true>), dim3((unsigned)(sa.n_sub * d.n_k_heads)), dim3(256), 0, st,
                           sa, (const Act *)x, (const Act *)conv_w, conv_on, g, beta, d.n_k_heads,
                           d.n_v_heads, d.l2_eps, ws);
    else
        hipLaunchKernelGGL((prep_kernel<D, Act, false>), dim3((unsigned)(sa.n_sub * d.n_k_heads)), dim3(256), 0, st,
                           sa, (const Act *)x, (const Act *)conv_w, conv_on, g, beta, d.n_k_heads,
                           d.n_v_heads, d.l2_eps, ws);
    em.mark(1);
    em.mark(2);
    const dim3 grid((D / kTileV) * d.n_v_heads, sa.n_seg);
    const bool pair = chain_ring2((int64_t)grid.x * grid.y);
    if (d.conv_silu && conv_on) {
        if (pair)
            hipLaunchKernelGGL((chain_kernel<D, Act, Out, true, 2>), grid, dim3(512), 0, st, sa,
                               (const Act *)x, (const Act *)conv_w, conv_on, d.n_k_heads,
                               d.n_v_heads, d.scale, ws, (Out *)o);
        else
            hipLaunchKernelGGL((chain_kernel<D, Act, Out, true, 3>), grid, dim3(512), 0, st, sa,
                               (const Act *)x, (const Act *)conv_w, conv_on, d.n_k_heads,
                               d.n_v_heads, d.scale, ws, (Out *)o);
    } else {
        if (pair)
            hipLaunchKernelGGL((chain_kernel<D, Act, Out, false, 2>), grid, dim3(512), 0, st, sa,
                               (const Act *)x, (const Act *)conv_w, conv_on, d.n_k_heads,
                               d.n_v_heads, d.scale, ws, (Out *)o);
        else
            hipLaunchKernelGGL((chain_kernel<D, Act, Out, false, 3>), grid, dim3(512), 0, st, sa,
                               (const Act *)x, (const Act *)conv_w, conv_on, d.n_k_heads,
                               d.n_v_heads, d.scale, ws, (Out *)o);
    }
    em.mark(3);
    em.mark(4);  // the conv window is written by the chain kernel
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
        hipLaunchKernelGGL((conv_step_kernel<Act, Out>), dim3((C / 8 + 255) / 256, (unsigned)nb),
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

int copy_to_host(void *host, const void *dev, size_t bytes, void *stream)
{
    return (int)hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream);
}

int copy_to_device(void *dev, const void *host, size_t bytes, void *stream)
{
    return (int)hipMemcpyAsync(dev, host, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
}

int stream_sync(void *stream) { return (int)hipStreamSynchronize((hipStream_t)stream); }

}  // namespace gdn
