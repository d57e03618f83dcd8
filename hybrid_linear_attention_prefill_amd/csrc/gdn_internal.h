// gdn_internal.h -- declarations shared by the host half (gdn_host.cpp) and the kernels
// (gdn_kernels.hip) of libgdn_prefill.so.  Not part of the public ABI.
//
// The host half compiles without ROCm: it reaches the device only through the launch_*
// functions below, which the HIP sources define.  So the same validation, grid arithmetic,
// checkpoint ring and state-file code can be built with a plain C++ compiler (and its
// sanitizers) against a host-memory stand-in for those functions, for CPU tests.
#pragma once
#include <cstddef>
#include <cstdint>

#include "gdn.h"

namespace gdn {

// Sequences handled by one launch.  A branch batch with more sequences is cut into
// launches of at most this many, issued in order on the caller's stream.
constexpr int kMaxSegPerLaunch = 32;
constexpr int kC = GDN_SUB_CHUNK;  // 64 rows per sub-chunk
constexpr int kTileV = 16;         // d_v columns of the state owned by one chain workgroup
// A lower-triangular 64x64 factor (Tinv or M) is stored as the MFMA A fragments that the chain
// kernel's waves load: (row tile w, 32-wide K step kb) for (0,0) (1,0) (2,0) (2,1) (3,0) (3,1),
// each 64 lanes x 8 fp16.  Lane l holds row 16w + l%16; its element e is column
// 32kb + 16(e/4) + 4(l/16) + e%4 (the K order of the step is permuted; the chain kernel
// stores the matching B operand rows in the same order).
constexpr int kTriFrags = 6;
constexpr int kPackedTri = kTriFrags * 64 * 8;

// One sequence of a launch: rows [row0, row0 + n) of x / g / beta / o, continued from
// (S_in, win_in) and finished into (S_out, win_out).  sub0 is the index of its first
// sub-chunk in the launch's workspace.
struct Seg {
    int64_t row0;
    int32_t n;
    int32_t sub0;
    const float *S_in;
    const void *win_in;
    float *S_out;
    void *win_out;
};

struct SegArgs {
    int32_t n_seg;
    int32_t n_sub;  // total sub-chunks of the launch
    Seg seg[kMaxSegPerLaunch];
};

// Workspace carved for one launch (device pointers).
// The fp16 arrays are held as raw 16-bit words here (the host half has no fp16 type); the
// kernels read and write them as _Float16.
struct Workspace {
    uint16_t *Qh;  // [n_sub][Hk][64*d]  normalised q, fp16, in MFMA A-fragment order
    uint16_t *Kh;  // [n_sub][Hk][64*d]  normalised k, likewise: fragment (w, kb) lane l holds
                   //                    row 16w + l%16, columns 32kb + 8(l/16) .. +7
    uint16_t *Tm;  // [n_sub][Hv][kPackedTri] (I + A)^-1 fragments, fp16 (order above)
    uint16_t *Mm;  // [n_sub][Hv][kPackedTri] lower(Q K^T) * decay fragments, fp16 (order above)
    float *Fac;    // [n_sub][Hv][4][64]  per row: beta, beta*gamma, gamma, exp(G_n - G) (fp32)
};

// One sequence of a decode launch: its input row, state, window and outputs (device).
struct DecodeSeq {
    const void *x;       // [C] the token's pre-conv row
    const float *S_in;   // [Hv][d_k][d_v]
    float *S_out;        // may equal S_in
    const void *win;     // [W-1][C] the window before the step (null without conv)
    void *win_out;       // [W-1][C] the window after the step, written by the step itself;
                         // null when the shift runs as a separate kernel (in-place windows)
    const float *g;      // [Hv]
    const float *beta;   // [Hv]
    void *o;             // [Hv][d_v]
};

struct DecodeArgs {
    int32_t n;
    DecodeSeq seq[kMaxSegPerLaunch];
};

// One sequence of an attention launch (device pointers): query rows pos0 .. pos0 + T - 1, keys
// and values 0 .. pos0 + T - 1 of its caches.  tile0 is its first row tile in the launch.
struct AttnSeq {
    const void *q;  // [T][Hq][D]
    const void *k;  // [pos0 + T][Hkv][D]
    const void *v;  // [pos0 + T][Hkv][D]
    void *o;        // [T][Hq][D]
    int64_t pos0, T;
    int32_t tile0;
};

struct AttnArgs {
    int32_t n;
    AttnSeq seq[kMaxSegPerLaunch];
};

// Query heads and 16-row tiles one attention workgroup covers: HW heads of one key head, each
// over 8 / HW row tiles (HW = min(Hq / Hkv, 8)).
inline int attn_heads_per_wg(int Hq, int Hkv) { return Hq / Hkv < 8 ? Hq / Hkv : 8; }

size_t workspace_bytes(const gdn_desc &d, int64_t n_sub);
Workspace carve_workspace(const gdn_desc &d, int64_t n_sub, void *base);

// Launchers (gdn_kernels.hip).  Return 0 or a hipError_t value.
// events: optional array of 2*n_kernels hipEvent_t recorded around each kernel (may be null).
int launch_prefill(const gdn_desc &d, const SegArgs &sa, const void *x, const void *conv_w,
                   const float *g, const float *beta, void *o, const Workspace &ws,
                   void *stream, void *const *events = nullptr, int n_events = 0);
// One decode step of da.n sequences (state and outputs), then the window shift of each
// sequence (window_out = rows 1 .. W-1 of window_in ++ x) when windows are given in `win`.
int launch_decode(const gdn_desc &d, const DecodeArgs &da, const SegArgs &win, const void *x,
                  const void *conv_w, void *stream);
int launch_conv_step(const gdn_desc &d, const void *x, const void *conv_w, void *window, void *y,
                     int64_t T, void *stream);
// y[T][N] = x[T][K] w[N][K]^T, bf16 in, fp32 accumulation, y in out_dtype (gdn_linear.hip).
int launch_linear(int64_t T, int K, int N, const void *x, const void *w, void *y, int out_dtype,
                  void *stream);
// Causal attention of aa.n sequences; c2 = scale * log2(e) (gdn_attention.hip).
int launch_attention(const AttnArgs &aa, int n_tiles, int Hq, int Hkv, int D, int HW, float c2,
                     int out_dtype, void *stream);
int launch_zero(void *p, size_t bytes, void *stream);
int launch_copy(void *dst, const void *src, size_t bytes, void *stream);
// Copies between device memory and host memory on `stream`, and a wait for the stream.
int copy_to_host(void *host, const void *dev, size_t bytes, void *stream);
int copy_to_device(void *dev, const void *host, size_t bytes, void *stream);
int stream_sync(void *stream);

}  // namespace gdn
