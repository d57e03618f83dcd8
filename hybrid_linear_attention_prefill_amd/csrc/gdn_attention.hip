// gdn_attention.hip -- causal prefill attention for the full-attention layers of a hybrid model:
// bf16 q / K / V, fp32 softmax and accumulation, on gfx950 MFMA.
//
// The pages run these layers as split-K flash attention: key positions are cut into splits of
// 256, the softmax is kept online, and the splits are merged in an order fixed by absolute
// position alone, so that any way of cutting a prompt into calls (or of grouping branches)
// gives the same bits ("Long context and sessions", section "The KV cache").  Here each query
// row folds its splits into a running (max, sum, accumulator) in ascending split order, one
// split per update: the split's largest score joins the running max, the running sum and
// accumulator are rescaled by exp(old max - new max), and the split's exponentials, rounded to
// bf16, are added with their value rows.  Split boundaries are absolute multiples of 256 and
// every row's arithmetic is the same whichever call, tile or lane it lands in.  Keys past a
// row's own position are masked to an exact zero weight, and keys past the cache end read as
// zero, so every block of a workgroup's last split can be run whole: a block masked for every
// row adds exact zeros (x + 0 and x * 1 are exact).
//
// Workgroup: 8 waves, each owning 16 query rows of one query head; the waves share the key
// head, so one 64-key block of K or V staged in LDS serves all of them.  For each split the
// waves first form S^T = K Q^T for its 256 keys (16 x 256 scores per wave, in registers), then
// the softmax update, then O^T += V^T P^T.  Both products put a query row in lane % 16, so the
// row statistics and the rescaling stay inside a lane.
//
// Staging: a split is eight 64-key blocks (its four K blocks, then its four V blocks), and
// block e of a split lives in LDS slot e mod 4, four separate arrays, so every read names a
// slot known at compile time.  The blocks go in pairs: while a pair is multiplied, the next
// pair is copied into the two other slots straight from global memory (buffer loads with the
// LDS bit: no registers, no LDS write instructions); then each wave waits for its own copies
// and the workgroup meets at a barrier, four times a split.  The compiler tells the four slots
// apart, so the products' LDS reads never wait for the copies bound for the other two.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr int kSplit = 256;  // key positions per split
constexpr int kBlk = 64;     // keys per LDS block
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// An LDS block holds 64 key rows of D bf16 (R = D / 8 chunks of 16 bytes per row), in one of two
// layouts of the same size; in both, every fragment address is one per-lane base plus a
// compile-time offset.
//  - V blocks: each row padded by one chunk, chunk c of row t at slot t (R + 1) + c, so rows t
//    and t + 1 start one chunk apart in the 256-byte bank window (the transposed reads below).
//  - K blocks: rows in pairs, chunk c of row t at slot (t / 2)(2 R + 2) + (t mod 2) R + c, so
//    rows 2 s and 2 s + 1 start at the same even chunk of the window and consecutive pairs two
//    chunks apart.  A 16-byte read serves its 64 lanes in four passes of 16, lanes 0-7 with
//    24-31 and 8-15 with 16-23 (and the same in the upper half): in a K fragment read those
//    are 8 even keys of one d-chunk with 8 odd keys of the next, which then fill the 16
//    chunk slots of the window.  (With padded rows an even and an odd key row meet in the same
//    slot: two-way conflicts, half of the LDS cycles of the reads.)
template <int D>
constexpr int kRowChunks = D / 8 + 1;
template <int D>
constexpr int kSlotChunks = kBlk * kRowChunks<D>;
template <int D>
constexpr int kPairChunks = 2 * (D / 8) + 2;  // one pair of K rows
template <int D>
__device__ __forceinline__ int k_row_start(int t)
{
    return (t >> 1) * kPairChunks<D> + (t & 1) * (D / 8);
}

// Key order inside a 16-key MFMA tile: row r of the tile is key sigma(r) = 2 (r mod 8) + r / 8.
// With it the 16 rows of a K fragment read have distinct residues mod 16 (no bank conflict),
// and the 8 rows each half-wave touches in a transposed V read are all even or all odd, so
// together with the two chunks per row they also fill 16 distinct slots.
__device__ __forceinline__ int sigma(int r) { return ((r & 7) << 1) | (r >> 3); }

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// K fragment (A operand of S^T = K Q^T) for tile q4 and d-step ks: lane (r = lane % 16, g)
// holds K[16 q4 + sigma(r)][32 ks + 8 g .. + 7].  kbase = the lane's slot offset of
// (sigma(r), g) in the paired-row layout; 16 rows are 8 pairs.
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const u32x4 *slot, int kbase, int q4, int ks)
{
    return __builtin_bit_cast(bf16x8, slot[kbase + 8 * q4 * kPairChunks<D> + 4 * ks]);
}

// V^T fragment (A operand of O^T = V^T P^T) for output columns 16 ct .. + 15 and the 32 keys
// of tiles 2 kb, 2 kb + 1 of a block: lane (col m = lane % 16, g) holds V[key][16 ct + m] for
// the keys 32 kb + sigma(4 g + e) and 32 kb + 16 + sigma(4 g + e), e = 0..3, the keys whose
// softmax weights the lane holds in the S^T layout.  ds_read_b64_tr_b16 gives output lane i of a
// 16-lane group element i % 4 of the 8-byte reads of lanes 4 e + i / 4 (e = 0..3); lane 4 a + b
// reads columns 16 ct + 4 b .. + 3 of key row 32 kb + sigma(4 g + a), so output lane i gets
// column 16 ct + i of those four rows.  vbase = the lane's byte offset for ct = kb = 0.
template <int D>
__device__ __forceinline__ bf16x8 v_frag(const u32x4 *slot, int vbase, int ct, int kb)
{
    typedef __attribute__((address_space(3))) short4_t lds_short4;
    const char *b = (const char *)slot + vbase + 32 * ct + 512 * kb * kRowChunks<D>;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)b);
    const short4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(b + 256 * kRowChunks<D>));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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
    const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *(u32x2 *)p = __builtin_bit_cast(u32x2, h);
}

typedef __attribute__((address_space(3))) void lds_void;

// A block's kSlotChunks<D> 16-byte chunks are filled by kNGI copy instructions of 64 lanes
// (lane i of instruction gi fills chunk 64 gi + i); wave w issues instructions w, w + 8, ...
// below kNGI: kJ of them, or kJ - 1 in waves past kNGI mod 8.
template <int D>
constexpr int kNGI = kSlotChunks<D> / 64;
template <int D>
constexpr int kJ = (kNGI<D> + kWaves - 1) / kWaves;
static_assert(kSlotChunks<128> % 64 == 0 && kSlotChunks<256> % 64 == 0, "whole copy instructions");

// Byte offset, from the block's first key, of what chunk p of a slot holds: key row and 16-byte
// column in the paired-row (K) or padded-row (V) layout; pad chunks take column 0 of their row.
template <int D>
__device__ __forceinline__ uint32_t dma_off(int p, bool isv, int Hkv, int kvh)
{
    constexpr int R = D / 8;
    int row, c;
    if (isv) {
        row = p / (R + 1);
        c = p % (R + 1);
        if (c == R) c = 0;
    } else {
        const int pair = p / kPairChunks<D>, q = p % kPairChunks<D>;
        row = 2 * pair + (q >= R && q < 2 * R ? 1 : 0);
        c = q < R ? q : (q < 2 * R ? q - R : 0);
    }
    if (row > kBlk - 1) row = kBlk - 1;  // offsets of copies a wave does not issue
    return (uint32_t)(((row * Hkv + kvh) * D + 8 * c) * 2);
}

// One 16-byte-per-lane copy from a buffer resource straight into 1 KB of LDS at dst (lane i's
// 16 bytes at dst + 16 i); reads outside the resource's range give zeros.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, u32x4 *dst, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, off, 0, 0, 0);
}

template <int D, typename Out>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a, int Hq, int Hkv, int HW,
                                                        float c2)
{
    __shared__ u32x4 slot0[kSlotChunks<D>], slot1[kSlotChunks<D>], slot2[kSlotChunks<D>],
        slot3[kSlotChunks<D>];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int RW = kWaves / HW;  // 16-row tiles per workgroup
    const int R = Hq / Hkv;

    // heavier (later) row tiles first; within a tile the head groups are adjacent, so that
    // consecutive workgroups (which go to different XCDs) take different key heads
    const int n_groups = Hkv * (Hq / Hkv / HW);
    const int group = (int)blockIdx.x % n_groups;
    const int tile = (int)(gridDim.x / n_groups) - 1 - (int)blockIdx.x / n_groups;
    int s = 0;
    for (int i = 1; i < a.n; ++i)
        if (a.seq[i].tile0 <= tile) s = i;
    const AttnSeq &sq = a.seq[s];
    const int64_t T = sq.T, pos0 = sq.pos0, L = pos0 + T;
    const int64_t t0 = (int64_t)(tile - sq.tile0) * 16 * RW;
    const int groups_per_kv = R / HW;
    const int kvh = group / groups_per_kv;
    const int h = kvh * R + (group % groups_per_kv) * HW + wave % HW;
    const int64_t tw = t0 + 16 * (wave / HW);  // this wave's first row
    const int64_t t_end = t0 + 16 * RW < T ? t0 + 16 * RW : T;
    const int64_t p_last = pos0 + t_end - 1;   // last valid row of the workgroup
    const int ns = (int)(p_last / kSplit) + 1;
    const int64_t trow = tw + li, prow = pos0 + trow;

    const uint16_t *kp = (const uint16_t *)sq.k, *vp = (const uint16_t *)sq.v;
    uint32_t offk[kJ<D>], offv[kJ<D>];  // this lane's copy offsets, the same for every block
#pragma unroll
    for (int i = 0; i < kJ<D>; ++i) {
        const int p = 64 * (wave + kWaves * i) + lane;
        offk[i] = dma_off<D>(p, false, Hkv, kvh);
        offv[i] = dma_off<D>(p, true, Hkv, kvh);
    }
    const int kbase = k_row_start<D>(sigma(li)) + g;
    const int j4 = lane & 15;
    const int vbase = 16 * sigma(4 * g + j4 / 4) * kRowChunks<D> + 8 * (j4 % 4);

    // q fragments of this lane's row (zero past T): B operand, lane (row, g) holds d 32 ks + 8 g ..
    bf16x8 qf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
        qf[ks] = trow < T ? __builtin_bit_cast(
                                bf16x8, *(const u32x4 *)((const uint16_t *)sq.q +
                                                         (trow * Hq + h) * D + 32 * ks + 8 * g))
                          : bf16x8{};

    f32x4 acc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the row sum of the (rounded) weights rides along as one more output tile against a
    // column of ones: the MFMA sums the 32 keys of a step, every lane gets its row's sum
    f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
    float m = -__builtin_inff();
    const int64_t p_wave = pos0 + tw;  // the wave's first (smallest) row position

    // Block q = 8 j + e: e < 4 the K block e of split j, else its V block e - 4, into slot
    // q mod 4 (keys past the cache end read as zero); nothing past the last split.
    auto dma = [&](u32x4 *slot, int q) {
        const int j = q >> 3, e = q & 7;
        if (j >= ns) return;
        const bool isv = e >= 4;
        const int64_t key0 = (int64_t)kSplit * j + kBlk * (e & 3);
        const int64_t nk = key0 < L ? (L - key0 < kBlk ? L - key0 : kBlk) : 0;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((isv ? vp : kp) + key0 * Hkv * D), 0, (int)(nk * Hkv * D * 2), kRsrcWord3);
#pragma unroll
        for (int i = 0; i < kJ<D>; ++i) {
            const int gi = wave + kWaves * i;
            if (gi < kNGI<D>) copy_to_lds(r, slot + 64 * gi, isv ? offv[i] : offk[i]);
        }
    };
    // this wave's copies have landed; then the workgroup meets (no fence: the copies are the
    // only memory traffic of the loop, and every LDS read of a pair is consumed before it)
    auto meet = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    dma(slot0, 0);
    dma(slot1, 1);
    meet();

    for (int j = 0; j < ns; ++j) {
        f32x4 S[kSplit / 16];  // S^T tiles: lane (row li, g) holds keys 16 kt + sigma(4 g + i)
        auto kstep = [&](const u32x4 *slot, int kc) {
            // fragments of d-step ks + 1 are read while step ks multiplies
            bf16x8 kf[2][4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) kf[0][q4] = k_frag<D>(slot, kbase, q4, 0);
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                if (ks + 1 < D / 32)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        kf[(ks + 1) & 1][q4] = k_frag<D>(slot, kbase, q4, ks + 1);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    S[4 * kc + q4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        kf[ks & 1][q4], qf[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[4 * kc + q4],
                        0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        const int q0 = 8 * j;
        dma(slot2, q0 + 2);
        dma(slot3, q0 + 3);
        kstep(slot0, 0);
        kstep(slot1, 1);
        meet();
        dma(slot0, q0 + 4);
        dma(slot1, q0 + 5);
        kstep(slot2, 2);
        kstep(slot3, 3);
        meet();

        // softmax update for split j (scores in units of log2: s * c2).  Key 16 kt + sigma(4 g
        // + i) of the split is live for this row when it is at most lim, the row's own
        // position; when every key of the split is at or below every row of the wave, nothing
        // is masked.
        const int64_t key_base = (int64_t)kSplit * j;
        const int64_t rel = prow - key_base;
        const int lim = rel < kSplit - 1 ? (int)rel : kSplit - 1;
        const bool full = p_wave - key_base >= kSplit - 1;
        float mx = -__builtin_inff();
        if (full) {
#pragma unroll
            for (int kt = 0; kt < kSplit / 16; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kt][i]);
        } else {
            int sg[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sg[i] = sigma(4 * g + i);
#pragma unroll
            for (int kt = 0; kt < kSplit / 16; ++kt) {
                const int lk = lim - 16 * kt;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (sg[i] > lk) S[kt][i] = -__builtin_inff();
                    mx = fmaxf(mx, S[kt][i]);
                }
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx * c2);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) acc[ct] *= alpha;

        // weights of the 32 keys 32 kb .. in the lane's key order, rounded to bf16 (a masked
        // key's -inf gives exactly 0)
        auto weights = [&](int kb) {
            bf16x8 pk;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pk[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S[2 * kb + e / 4][e % 4], c2, -m_new));
            return pk;
        };
        auto vstep = [&](const u32x4 *slot, int vc) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const bf16x8 pk = weights(2 * vc + kb2);
                lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk, lsum, 0, 0, 0);
                // V^T fragments of columns ct + 1 .. ct + 2 in flight while ct multiplies
                bf16x8 vf[4];
                vf[0] = v_frag<D>(slot, vbase, 0, kb2);
                vf[1] = v_frag<D>(slot, vbase, 1, kb2);
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    if (ct + 2 < D / 16) vf[(ct + 2) & 3] = v_frag<D>(slot, vbase, ct + 2, kb2);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ct & 3], pk, acc[ct], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        dma(slot2, q0 + 6);
        dma(slot3, q0 + 7);
        vstep(slot0, 0);
        vstep(slot1, 1);
        meet();
        dma(slot0, q0 + 8);
        dma(slot1, q0 + 9);
        vstep(slot2, 2);
        vstep(slot3, 3);
        meet();
    }

    if (trow < T) {
        const float inv = 1.0f / lsum[0];
        Out *orow = (Out *)sq.o + (trow * Hq + h) * D;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) store4<Out>(orow + 16 * ct + 4 * g, acc[ct] * inv);
    }
}

template <int D>
int launch_d(const AttnArgs &aa, int n_tiles, int Hq, int Hkv, int HW, float c2, int out_dtype,
             hipStream_t st)
{
    const dim3 grid((unsigned)(n_tiles * Hkv * (Hq / Hkv / HW)));
    if (out_dtype == GDN_BF16)
        hipLaunchKernelGGL((attn_kernel<D, uint16_t>), grid, dim3(kThreads), 0, st, aa, Hq, Hkv,
                           HW, c2);
    else
        hipLaunchKernelGGL((attn_kernel<D, float>), grid, dim3(kThreads), 0, st, aa, Hq, Hkv, HW,
                           c2);
    return (int)hipGetLastError();
}

}  // namespace

int launch_attention(const AttnArgs &aa, int n_tiles, int Hq, int Hkv, int D, int HW, float c2,
                     int out_dtype, void *stream)
{
    (void)hipGetLastError();
    if (n_tiles == 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    return D == 128 ? launch_d<128>(aa, n_tiles, Hq, Hkv, HW, c2, out_dtype, st)
                    : launch_d<256>(aa, n_tiles, Hq, Hkv, HW, c2, out_dtype, st);
}

}  // namespace gdn
