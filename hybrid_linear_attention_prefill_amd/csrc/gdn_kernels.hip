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

__device__ __forceinline__ int find_seg(const SegArgs &sa, int sub)
{
    int s = 0;
    for (int i = 1; i < sa.n_seg; ++i)
        if (sa.seg[i].sub0 <= sub) s = i;
    return s;
}

// ------------------------------------------------------------------------------------------
// prep_kernel: state-independent factors of one (sub-chunk, key head).
// ------------------------------------------------------------------------------------------
template <int D, typename Act>
__global__ __launch_bounds__(256) void prep_kernel(SegArgs sa, const Act *__restrict__ x,
                                                   const Act *__restrict__ conv_w, int conv_on,
                                                   int silu, const float *__restrict__ g,
                                                   const float *__restrict__ beta, int Hk, int Hv,
                                                   float eps, Workspace ws)
{
    constexpr int NCH = 2 * D;          // q and k channels of one key head
    constexpr int TPC = 256 / NCH;      // threads per channel
    constexpr int RPT = kC / TPC;       // rows per thread
    constexpr int YS = NCH + 4;         // fp32 row stride of the conv output
    constexpr int HS = D + 8;           // fp16 row stride of q, k
    constexpr int AS = kC + 1;          // fp32 row stride of A, Tinv
    constexpr int YWORDS = kC * YS;
    constexpr int AWORDS = 2 * kC * AS + 16 * kC;
    __shared__ __attribute__((aligned(16))) float ybuf[YWORDS > AWORDS ? YWORDS : AWORDS];
    __shared__ __attribute__((aligned(16))) _Float16 q16[kC * HS];
    __shared__ __attribute__((aligned(16))) _Float16 k16[kC * HS];
    __shared__ float inv_n[2][kC];
    __shared__ float Gs[kC], bs[kC];
    float *const As = ybuf;              // after the norms, ybuf holds A, Tinv and a rhs block
    float *const Ts = ybuf + kC * AS;
    float *const Rs = ybuf + 2 * kC * AS;

    const int sub = blockIdx.x, kh = blockIdx.y;
    const int s = find_seg(sa, sub);
    const int64_t seg_row0 = sa.seg[s].row0;
    const int seg_n = sa.seg[s].n;
    const Act *win = (const Act *)sa.seg[s].win_in;
    const int r_base = (sub - sa.seg[s].sub0) * kC;  // sequence-local first row
    const int nv = min(kC, seg_n - r_base);          // valid rows
    const int C = 2 * Hk * D + Hv * D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // 1. causal conv of the q | k channels (fp32 accumulate), rows past the end are zero
    {
        const int lc = tid % NCH, part = tid / NCH;
        const int ch = (lc < D) ? (kh * D + lc) : (Hk * D + kh * D + (lc - D));
        const int ra = part * RPT;
        auto xt = [&](int r) -> float {  // sub-chunk-local row, may be -3..-1
            const int sr = r_base + r;
            if (sr < 0) return to_f32(win[(3 + sr) * C + ch]);
            if (sr >= seg_n) return 0.f;
            return to_f32(x[(seg_row0 + sr) * C + ch]);
        };
        if (conv_on) {
            const float w0 = to_f32(conv_w[ch * 4 + 0]), w1 = to_f32(conv_w[ch * 4 + 1]);
            const float w2 = to_f32(conv_w[ch * 4 + 2]), w3 = to_f32(conv_w[ch * 4 + 3]);
            float a0 = xt(ra - 3), a1 = xt(ra - 2), a2 = xt(ra - 1);
            for (int r = ra; r < ra + RPT; ++r) {
                const float a3 = xt(r);
                float y = w0 * a0 + w1 * a1 + w2 * a2 + w3 * a3;
                if (silu) y = y / (1.f + expf(-y));
                ybuf[r * YS + lc] = (r < nv) ? y : 0.f;
                a0 = a1;
                a1 = a2;
                a2 = a3;
            }
        } else {
            for (int r = ra; r < ra + RPT; ++r) ybuf[r * YS + lc] = (r < nv) ? xt(r) : 0.f;
        }
    }
    __syncthreads();

    // 2. inverse norms 1/sqrt(|y|^2 + eps) of each q and k row (0 for rows past the end)
    {
        const int p = tid >> 1, half = tid & 1;
        const int r = p >> 1, which = p & 1;
        const float *src = ybuf + r * YS + which * D + half * (D / 2);
        float ss = 0.f;
        for (int i = 0; i < D / 2; ++i) ss += src[i] * src[i];
        ss += __shfl_xor(ss, 1);
        if (half == 0) inv_n[which][r] = (r < nv) ? 1.0f / sqrtf(ss + eps) : 0.f;
    }
    __syncthreads();

    // 3. normalised q, k as fp16 into LDS and the workspace
    {
        _Float16 *Qg = ws.Qh + ((int64_t)sub * Hk + kh) * kC * D;
        _Float16 *Kg = ws.Kh + ((int64_t)sub * Hk + kh) * kC * D;
        for (int e = tid; e < kC * D; e += 256) {
            const int r = e / D, i = e % D;
            const _Float16 qv = (_Float16)(ybuf[r * YS + i] * inv_n[0][r]);
            const _Float16 kv = (_Float16)(ybuf[r * YS + D + i] * inv_n[1][r]);
            q16[r * HS + i] = qv;
            k16[r * HS + i] = kv;
            Qg[e] = qv;
            Kg[e] = kv;
        }
    }
    __syncthreads();

    // 4. K K^T and Q K^T, row tile `wave`, column tiles j <= wave
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

    // 5. per value head of this key head's group
    const int group = Hv / Hk;
    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        if (wave == 0) {  // cumulative log decay (inclusive scan), beta; past the end: 0
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
            ws.Gc[((int64_t)sub * Hv + h) * kC + r] = gv;
        }
        __syncthreads();

        // A (fp32, LDS) and M (fp16, workspace), full 64x64 with zeros above the diagonal
        {
            _Float16 *Mg = ws.Mm + ((int64_t)sub * Hv + h) * kC * kC;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
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
                    Ts[r * AS + c] = 0.f;
                    Mg[r * kC + c] = (_Float16)m;
                }
            }
        }
        __syncthreads();

        // Tinv = (I + A)^-1.  Phase 1: the four diagonal 16x16 blocks, one per 16 lanes of
        // wave 0, by forward substitution (lane = 16 b + column).
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
        }
        __syncthreads();
        // Phase 2: row blocks b = 1..3: Tinv[b, <b] = L_bb^-1 (-A[b, <b] Tinv[<b, <b]).
        for (int b = 1; b < 4; ++b) {
            {
                const int r = tid / 16, c0 = tid % 16;
                for (int m = 0; m < b; ++m) {
                    const int c = c0 + 16 * m;
                    float acc = 0.f;
                    for (int i = 0; i < 16 * b; ++i) acc -= As[(16 * b + r) * AS + i] * Ts[i * AS + c];
                    Rs[r * kC + c] = acc;
                }
            }
            __syncthreads();
            {
                const int r = tid / 16, c0 = tid % 16;
                for (int m = 0; m < b; ++m) {
                    const int c = c0 + 16 * m;
                    float acc = 0.f;
                    for (int i = 0; i < 16; ++i)
                        acc += Ts[(16 * b + r) * AS + 16 * b + i] * Rs[i * kC + c];
                    Ts[(16 * b + r) * AS + c] = acc;
                }
            }
            __syncthreads();
        }
        {
            _Float16 *Tg = ws.Tm + ((int64_t)sub * Hv + h) * kC * kC;
            for (int e = tid; e < kC * kC; e += 256) Tg[e] = (_Float16)Ts[(e / kC) * AS + e % kC];
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------
// chain_kernel: the serial walk of one (d_v tile, value head, sequence) over its sub-chunks.
// ------------------------------------------------------------------------------------------
template <int D, typename Act, typename Out>
__global__ __launch_bounds__(256) void chain_kernel(SegArgs sa, const Act *__restrict__ x,
                                                    const Act *__restrict__ conv_w, int conv_on,
                                                    int silu, const float *__restrict__ beta,
                                                    int Hk, int Hv, float scale, Workspace ws,
                                                    Out *__restrict__ o)
{
    constexpr int HS = D + 8;     // fp16 row stride of q, k
    constexpr int TS = kC + 8;    // fp16 row stride of Tinv, M and of the transposed 64-row tiles
    constexpr int ST = D + 8;     // fp16 row stride of S^T
    constexpr int NT = D / 16;    // d_k tiles of the state
    constexpr int TPW = NT / 4;   // d_k tiles per wave
    __shared__ __attribute__((aligned(16))) _Float16 k16[kC * HS];
    __shared__ __attribute__((aligned(16))) _Float16 q16[kC * HS];
    __shared__ __attribute__((aligned(16))) _Float16 t16[kC * TS];
    __shared__ __attribute__((aligned(16))) _Float16 m16[kC * TS];
    __shared__ __attribute__((aligned(16))) _Float16 s16t[16 * ST];  // S^T, fp16 MFMA operand
    __shared__ __attribute__((aligned(16))) _Float16 rt[16 * TS];    // R^T
    __shared__ __attribute__((aligned(16))) _Float16 dt[16 * TS];    // D^T
    __shared__ __attribute__((aligned(16))) _Float16 ddt[16 * TS];   // (exp(G_n - G) D)^T
    __shared__ float Gs[kC], bs[kC];
    __shared__ float xv[(kC + 3) * 16];

    const int tile = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int64_t seg_row0 = sa.seg[s].row0;
    const int seg_n = sa.seg[s].n;
    const int sub0 = sa.seg[s].sub0;
    const Act *win = (const Act *)sa.seg[s].win_in;
    const float *S_in = sa.seg[s].S_in;
    float *S_out = sa.seg[s].S_out;
    const int kh = h / (Hv / Hk);
    const int C = 2 * Hk * D + Hv * D;
    const int c0 = tile * 16;
    const int vch = 2 * Hk * D + h * D + c0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane % 16, kg = lane / 16;

    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 1.f;
    if (conv_on) {
        w0 = to_f32(conv_w[(vch + col) * 4 + 0]);
        w1 = to_f32(conv_w[(vch + col) * 4 + 1]);
        w2 = to_f32(conv_w[(vch + col) * 4 + 2]);
        w3 = to_f32(conv_w[(vch + col) * 4 + 3]);
    }

    f32x4 S[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int kt = wave * TPW + t;
        half4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 16 * kt + 4 * kg + i;
            S[t][i] = S_in[((int64_t)h * D + k) * D + c0 + col];
            sv[i] = (_Float16)S[t][i];
        }
        *(half4 *)(s16t + col * ST + 16 * kt + 4 * kg) = sv;
    }

    const int nsub = (seg_n + kC - 1) / kC;
    for (int cl = 0; cl < nsub; ++cl) {
        const int sub = sub0 + cl;
        const int r_base = cl * kC;
        const int nv = min(kC, seg_n - r_base);
        {
            const _Float16 *Kg = ws.Kh + ((int64_t)sub * Hk + kh) * kC * D;
            const _Float16 *Qg = ws.Qh + ((int64_t)sub * Hk + kh) * kC * D;
            for (int e = tid; e < kC * D / 8; e += 256) {
                const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
                *(half8 *)(k16 + r * HS + cc) = *(const half8 *)(Kg + r * D + cc);
                *(half8 *)(q16 + r * HS + cc) = *(const half8 *)(Qg + r * D + cc);
            }
            const _Float16 *Tg = ws.Tm + ((int64_t)sub * Hv + h) * kC * kC;
            const _Float16 *Mg = ws.Mm + ((int64_t)sub * Hv + h) * kC * kC;
            for (int e = tid; e < kC * kC / 8; e += 256) {
                const int r = e / 8, cc = (e % 8) * 8;
                *(half8 *)(t16 + r * TS + cc) = *(const half8 *)(Tg + r * kC + cc);
                *(half8 *)(m16 + r * TS + cc) = *(const half8 *)(Mg + r * kC + cc);
            }
            if (tid < kC) {
                Gs[tid] = ws.Gc[((int64_t)sub * Hv + h) * kC + tid];
                bs[tid] = (tid < nv) ? beta[(seg_row0 + r_base + tid) * Hv + h] : 0.f;
            }
            for (int e = tid; e < (kC + 3) * 16; e += 256) {
                const int rr = e / 16, cc = e % 16;
                const int sr = r_base + rr - 3;  // sequence-local row
                float v = 0.f;
                if (sr >= 0) {
                    if (sr < seg_n) v = to_f32(x[(seg_row0 + sr) * C + vch + cc]);
                } else if (conv_on) {
                    v = to_f32(win[(3 + sr) * C + vch + cc]);
                }
                xv[e] = v;
            }
        }
        __syncthreads();

        // X = K S and P = Q S for row tile `wave`
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) {
            const int off = 32 * kb + 8 * kg;
            const half8 b = *(const half8 *)(s16t + col * ST + off);
            X = mfma16(*(const half8 *)(k16 + (16 * wave + col) * HS + off), b, X);
            P = mfma16(*(const half8 *)(q16 + (16 * wave + col) * HS + off), b, P);
        }

        // R = diag(beta) (V - diag(gamma) X);  the state part of O is gamma Q S
        f32x4 Ob;
        {
            half4 rv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * wave + 4 * kg + i;
                const float *xr = xv + r * 16 + col;  // rows r .. r+3 of (halo ++ rows)
                float v = w0 * xr[0] + w1 * xr[16] + w2 * xr[32] + w3 * xr[48];
                if (silu && conv_on) v = v / (1.f + expf(-v));
                const float gam = expf(Gs[r]);
                rv[i] = (_Float16)(bs[r] * (v - gam * X[i]));
                Ob[i] = gam * P[i];
            }
            *(half4 *)(rt + col * TS + 16 * wave + 4 * kg) = rv;
        }
        __syncthreads();

        // D = Tinv R (Tinv lower triangular: row tile w needs columns < 16 (w + 1))
        f32x4 Dl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb == 0 || wave >= 2) {
                const int off = 32 * kb + 8 * kg;
                Dl = mfma16(*(const half8 *)(t16 + (16 * wave + col) * TS + off),
                            *(const half8 *)(rt + col * TS + off), Dl);
            }
        }
        const float Gn = Gs[kC - 1];
        {
            half4 dv, ddv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * wave + 4 * kg + i;
                dv[i] = (_Float16)Dl[i];
                ddv[i] = (_Float16)(expf(Gn - Gs[r]) * Dl[i]);
            }
            *(half4 *)(dt + col * TS + 16 * wave + 4 * kg) = dv;
            *(half4 *)(ddt + col * TS + 16 * wave + 4 * kg) = ddv;
        }
        __syncthreads();

        // O = scale (gamma Q S + M D)
        {
            f32x4 Oa = Ob;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb == 0 || wave >= 2) {
                    const int off = 32 * kb + 8 * kg;
                    Oa = mfma16(*(const half8 *)(m16 + (16 * wave + col) * TS + off),
                                *(const half8 *)(dt + col * TS + off), Oa);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * wave + 4 * kg + i;
                if (r < nv) store_out(o + ((seg_row0 + r_base + r) * Hv + h) * D + c0 + col, scale * Oa[i]);
            }
        }

        // S' = gamma_n S + K^T (exp(G_n - G) D)
        {
            const float gn = expf(Gn);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int kt = wave * TPW + t;
                f32x4 acc = S[t] * gn;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int off = 32 * kb + 8 * kg;
                    half8 a;
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = k16[(off + e) * HS + 16 * kt + col];
                    acc = mfma16(a, *(const half8 *)(ddt + col * TS + off), acc);
                }
                S[t] = acc;
                half4 sv;
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[i] = (_Float16)acc[i];
                *(half4 *)(s16t + col * ST + 16 * kt + 4 * kg) = sv;
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int kt = wave * TPW + t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 16 * kt + 4 * kg + i;
            S_out[((int64_t)h * D + k) * D + c0 + col] = S[t][i];
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
    hipLaunchKernelGGL((chain_kernel<D, Act, Out>), dim3(D / kTileV, d.n_v_heads, sa.n_seg),
                       dim3(256), 0, st, sa, (const Act *)x, (const Act *)conv_w, conv_on,
                       d.conv_silu, beta, d.n_k_heads, d.n_v_heads, d.scale, ws, (Out *)o);
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
