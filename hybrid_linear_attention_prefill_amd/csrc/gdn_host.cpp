// gdn_host.cpp -- host half of libgdn_prefill.so: argument validation, the commit-grid
// arithmetic, state copies and the launch sequence.  It includes no ROCm header: the device
// is reached only through the launch_* functions of gdn_internal.h.  Every check runs before the first HIP
// call, so a refused call enqueues nothing and changes no state (the pages refuse invalid
// requests before any device work: PR "qwen3_5: run prompts that share prefixes once per
// prefix", sections "Test Plan" and "Test Result").
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "gdn_internal.h"

namespace gdn {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int64_t n_channels(const gdn_desc &d)
{
    return 2 * (int64_t)d.n_k_heads * d.d_k + (int64_t)d.n_v_heads * d.d_v;
}
static size_t act_size(const gdn_desc &d) { return d.act_dtype == GDN_BF16 ? 2 : 4; }
static size_t out_size(const gdn_desc &d) { return d.out_dtype == GDN_BF16 ? 2 : 4; }

size_t workspace_bytes(const gdn_desc &d, int64_t n_sub)
{
    const size_t qk = align256((size_t)n_sub * d.n_k_heads * kC * d.d_k * 2);
    const size_t tm = align256((size_t)n_sub * d.n_v_heads * kPackedTri * 2);
    const size_t gc = align256((size_t)n_sub * d.n_v_heads * 4 * kC * 4);
    return 2 * qk + 2 * tm + gc;
}

Workspace carve_workspace(const gdn_desc &d, int64_t n_sub, void *base)
{
    const size_t qk = align256((size_t)n_sub * d.n_k_heads * kC * d.d_k * 2);
    const size_t tm = align256((size_t)n_sub * d.n_v_heads * kPackedTri * 2);
    char *p = (char *)base;
    Workspace w;
    w.Qh = (uint16_t *)p;
    w.Kh = (uint16_t *)(p + qk);
    w.Tm = (uint16_t *)(p + 2 * qk);
    w.Mm = (uint16_t *)(p + 2 * qk + tm);
    w.Fac = (float *)(p + 2 * qk + 2 * tm);
    return w;
}

// Alignment the kernels' vector accesses need: 16 bytes for x, conv weights, conv windows,
// outputs and the workspace; 4 bytes for g, beta and S.
static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + nb && pb < pa + na;
}

// Memory of a state (S and window) as two ranges.
struct Ranges {
    const void *p[2];
    size_t n[2];
};
static Ranges ranges_of(const gdn_desc &d, const gdn_state *s)
{
    Ranges r;
    r.p[0] = s->S;
    r.n[0] = gdn_state_S_bytes(&d);
    r.p[1] = s->conv;
    r.n[1] = gdn_state_conv_bytes(&d);
    return r;
}
static bool states_overlap(const gdn_desc &d, const gdn_state *a, const gdn_state *b)
{
    const Ranges ra = ranges_of(d, a), rb = ranges_of(d, b);
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            if (overlap(ra.p[i], ra.n[i], rb.p[j], rb.n[j])) return true;
    return false;
}

// The buffers a prefill reads (x, g, beta, conv weights, the entry states) and writes (o, the
// workspace bytes it uses, the final states): a written buffer that overlaps any other would
// race with the kernels that read or write it, so such calls are refused (GDN_EALIAS).
// `n` rows of x, g, beta and o; entry and final states may be the same state (a commit in
// place), which the callers check apart.
static bool io_overlap(const gdn_desc &d, int64_t n, const void *x, const void *conv_w,
                       const float *g, const float *beta, const void *o, const void *ws,
                       size_t ws_used, const gdn_state *const *ins, int n_in,
                       const gdn_state *const *outs, int n_out)
{
    const int64_t C = n_channels(d);
    const size_t xb = (size_t)(n * C) * act_size(d), gb = (size_t)n * d.n_v_heads * 4;
    const size_t wb = d.conv_width > 0 ? (size_t)C * d.conv_width * act_size(d) : 0;
    const size_t ob = (size_t)n * d.n_v_heads * d.d_v * out_size(d);
    const void *rp[4] = {x, g, beta, conv_w};
    const size_t rn[4] = {xb, gb, gb, wb};
    const void *wp[2] = {o, ws};
    const size_t wn[2] = {ob, ws_used};
    for (int a = 0; a < 2; ++a) {
        for (int r = 0; r < 4; ++r)
            if (overlap(wp[a], wn[a], rp[r], rn[r])) return true;
        if (a == 0 && overlap(wp[0], wn[0], wp[1], wn[1])) return true;
        for (int k = 0; k < n_in + n_out; ++k) {
            const Ranges q = ranges_of(d, k < n_in ? ins[k] : outs[k - n_in]);
            for (int t = 0; t < 2; ++t)
                if (overlap(wp[a], wn[a], q.p[t], q.n[t])) return true;
        }
    }
    for (int k = 0; k < n_out; ++k) {
        const Ranges q = ranges_of(d, outs[k]);
        for (int t = 0; t < 2; ++t)
            for (int r = 0; r < 4; ++r)
                if (overlap(q.p[t], q.n[t], rp[r], rn[r])) return true;
    }
    return false;
}
static bool states_same(const gdn_state *a, const gdn_state *b)
{
    return a == b || (a->S == b->S && a->conv == b->conv);
}

static gdn_status check_state(const gdn_desc &d, const gdn_state *s)
{
    if (!s || !s->S || !aligned(s->S, 4)) return GDN_EINVAL;
    if (d.conv_width > 0 && (!s->conv || !aligned(s->conv, 16))) return GDN_EINVAL;
    if (s->pos < 0) return GDN_EINVAL;
    if (s->tag != gdn_desc_tag(&d)) return GDN_EMISMATCH;
    return GDN_OK;
}

// A state the library writes (init, capture, restore, fork targets): the copy and zero kernels
// move S in 4-byte words and the window in 16-byte pieces.
static gdn_status check_dst(const gdn_desc &d, const gdn_state *s)
{
    if (!s || !s->S || !aligned(s->S, 4)) return GDN_EINVAL;
    if (d.conv_width > 0 && (!s->conv || !aligned(s->conv, 16))) return GDN_EINVAL;
    return GDN_OK;
}

static gdn_status copy_state(const gdn_desc &d, const gdn_state *src, gdn_state *dst, void *stream)
{
    if (launch_copy(dst->S, src->S, gdn_state_S_bytes(&d), stream) != 0) return GDN_EDEVICE;
    if (d.conv_width > 0 &&
        launch_copy(dst->conv, src->conv, gdn_state_conv_bytes(&d), stream) != 0)
        return GDN_EDEVICE;
    return GDN_OK;
}

// Runs the kernels over `segs` (already validated), cutting them into launches of at most
// kMaxSegPerLaunch sequences.  Each launch reuses the workspace from its start; launches are
// ordered on the stream.
static gdn_status run_segments(const gdn_desc &d, const std::vector<Seg> &segs, const void *x,
                               const void *conv_w, const float *g, const float *beta, void *o,
                               void *ws, void *stream, void *const *events = nullptr,
                               int n_events = 0)
{
    for (size_t b = 0; b < segs.size(); b += kMaxSegPerLaunch) {
        SegArgs sa;
        std::memset(&sa, 0, sizeof(sa));
        const size_t e = std::min(segs.size(), b + (size_t)kMaxSegPerLaunch);
        int32_t sub = 0;
        for (size_t i = b; i < e; ++i) {
            Seg s = segs[i];
            s.sub0 = sub;
            sub += (s.n + kC - 1) / kC;
            sa.seg[sa.n_seg++] = s;
        }
        sa.n_sub = sub;
        if (sub == 0) continue;
        const Workspace w = carve_workspace(d, sub, ws);
        if (launch_prefill(d, sa, x, conv_w, g, beta, o, w, stream, b == 0 ? events : nullptr,
                           n_events) != 0)
            return GDN_EDEVICE;
    }
    return GDN_OK;
}

// Rows of one sequence per launch: the chain kernel addresses x and o of a sequence with 32-bit
// byte offsets, so a longer sequence is run as several chained launches, each starting at a
// multiple of 64 rows (which changes no bit of the result).
// The environment variable GDN_TEST_LAUNCH_ROWS (a positive multiple of 64) lowers the cap, so
// that tests can run the chained-launch path at small sizes; it is read on every call and never
// raises the cap.
static int64_t max_rows_per_launch(const gdn_desc &d)
{
    const int64_t row_bytes = std::max<int64_t>(n_channels(d) * (int64_t)act_size(d),
                                                (int64_t)d.n_v_heads * d.d_v * (int64_t)out_size(d));
    const int64_t rows = ((int64_t)INT32_MAX - 4 * row_bytes) / row_bytes;
    int64_t cap = (rows / kC) * kC;
    if (const char *e = std::getenv("GDN_TEST_LAUNCH_ROWS")) {
        char *end = nullptr;
        const long long v = std::strtoll(e, &end, 10);
        if (end != e && *end == '\0' && v > 0 && v % kC == 0 && v < cap) cap = v;
    }
    return cap;
}

// Largest per-launch sub-chunk count of `segs`.
static int64_t max_launch_subs(const std::vector<Seg> &segs)
{
    int64_t best = 0;
    for (size_t b = 0; b < segs.size(); b += kMaxSegPerLaunch) {
        int64_t sub = 0;
        for (size_t i = b; i < std::min(segs.size(), b + (size_t)kMaxSegPerLaunch); ++i)
            sub += (segs[i].n + kC - 1) / kC;
        best = std::max(best, sub);
    }
    return best;
}

// ---------------------------------------------------------------- state files

struct StateFileHeader {
    char magic[8];
    uint32_t version, header_bytes;
    int32_t n_k_heads, n_v_heads, d_k, d_v, conv_width, sub_chunk, grid, act_dtype;
    uint64_t tag, weights_hash;
    int64_t pos;
    uint64_t S_bytes, conv_bytes, payload_hash, header_hash;
};
static_assert(sizeof(StateFileHeader) == 104, "state file header layout");
static const char kStateMagic[8] = {'G', 'D', 'N', 'S', 'T', 'A', 'T', '1'};

static uint64_t fnv1a(uint64_t h, const void *p, size_t n)
{
    const unsigned char *c = (const unsigned char *)p;
    for (size_t i = 0; i < n; ++i) {
        h ^= c[i];
        h *= 1099511628211ull;
    }
    return h;
}
static const uint64_t kFnvBasis = 1469598103934665603ull;

static StateFileHeader make_header(const gdn_desc &d, int64_t pos, uint64_t weights_hash,
                                   size_t s_bytes, size_t c_bytes)
{
    StateFileHeader h;
    std::memset(&h, 0, sizeof(h));
    std::memcpy(h.magic, kStateMagic, 8);
    h.version = 1;
    h.header_bytes = (uint32_t)sizeof(StateFileHeader);
    h.n_k_heads = d.n_k_heads;
    h.n_v_heads = d.n_v_heads;
    h.d_k = d.d_k;
    h.d_v = d.d_v;
    h.conv_width = d.conv_width;
    h.sub_chunk = d.sub_chunk;
    h.grid = d.grid;
    h.act_dtype = d.act_dtype;
    h.tag = gdn_desc_tag(&d);
    h.weights_hash = weights_hash;
    h.pos = pos;
    h.S_bytes = s_bytes;
    h.conv_bytes = c_bytes;
    return h;
}

static gdn_status write_state_file(const gdn_desc &d, const void *S, const void *conv,
                                   int64_t pos, uint64_t weights_hash, const char *path)
{
    const size_t sb = gdn_state_S_bytes(&d), cb = gdn_state_conv_bytes(&d);
    StateFileHeader h = make_header(d, pos, weights_hash, sb, cb);
    h.payload_hash = fnv1a(fnv1a(kFnvBasis, S, sb), conv, cb);
    h.header_hash = fnv1a(kFnvBasis, &h, offsetof(StateFileHeader, header_hash));
    // a failed write must leave no file at `path`: remove the old one first
    if (std::remove(path) != 0 && errno != ENOENT) return GDN_EFILE;
    const std::string tmp = std::string(path) + ".tmp." + std::to_string((long)getpid());
    FILE *f = std::fopen(tmp.c_str(), "wb");
    if (!f) return GDN_EFILE;
    bool ok = std::fwrite(&h, sizeof(h), 1, f) == 1 && std::fwrite(S, 1, sb, f) == sb &&
              (cb == 0 || std::fwrite(conv, 1, cb, f) == cb);
    ok = std::fflush(f) == 0 && ok;
    ok = fsync(fileno(f)) == 0 && ok;
    ok = std::fclose(f) == 0 && ok;
    if (!ok || std::rename(tmp.c_str(), path) != 0) {
        std::remove(tmp.c_str());
        return GDN_EFILE;
    }
    return GDN_OK;
}

// Reads and verifies the file into host buffers S and conv (sized for `d`); nothing is written
// to S, conv or *pos unless every check passes.
static gdn_status read_state_file(const gdn_desc &d, void *S, void *conv, int64_t *pos,
                                  uint64_t weights_hash, const char *path)
{
    const size_t sb = gdn_state_S_bytes(&d), cb = gdn_state_conv_bytes(&d);
    FILE *f = std::fopen(path, "rb");
    if (!f) return GDN_EFILE;
    StateFileHeader h;
    std::vector<unsigned char> payload;
    gdn_status st = GDN_OK;
    if (std::fread(&h, sizeof(h), 1, f) != 1 || std::memcmp(h.magic, kStateMagic, 8) != 0 ||
        h.version != 1 || h.header_bytes != sizeof(h) ||
        h.header_hash != fnv1a(kFnvBasis, &h, offsetof(StateFileHeader, header_hash))) {
        st = GDN_EFILE;
    } else {
        const StateFileHeader want = make_header(d, h.pos, weights_hash, sb, cb);
        if (h.n_k_heads != want.n_k_heads || h.n_v_heads != want.n_v_heads || h.d_k != want.d_k ||
            h.d_v != want.d_v || h.conv_width != want.conv_width || h.sub_chunk != want.sub_chunk ||
            h.grid != want.grid || h.act_dtype != want.act_dtype || h.tag != want.tag ||
            h.weights_hash != want.weights_hash || h.S_bytes != sb || h.conv_bytes != cb) {
            st = GDN_EMISMATCH;
        } else if (h.pos < 0) {
            st = GDN_EFILE;
        } else {
            payload.resize(sb + cb);
            if (std::fread(payload.data(), 1, sb + cb, f) != sb + cb || std::fgetc(f) != EOF ||
                fnv1a(kFnvBasis, payload.data(), sb + cb) != h.payload_hash)
                st = GDN_EFILE;
        }
    }
    std::fclose(f);
    if (st) return st;
    std::memcpy(S, payload.data(), sb);
    if (cb) std::memcpy(conv, payload.data() + sb, cb);
    *pos = h.pos;
    return GDN_OK;
}

}  // namespace gdn

using namespace gdn;

extern "C" {

gdn_status gdn_desc_check(const gdn_desc *d)
{
    if (!d) return GDN_EINVAL;
    if (d->n_k_heads <= 0 || d->n_v_heads <= 0 || d->d_k <= 0 || d->d_v <= 0) return GDN_EINVAL;
    if (d->act_dtype != GDN_BF16 && d->act_dtype != GDN_F32) return GDN_EINVAL;
    if (d->out_dtype != GDN_BF16 && d->out_dtype != GDN_F32) return GDN_EINVAL;
    if (d->conv_silu != 0 && d->conv_silu != 1) return GDN_EINVAL;
    if (!std::isfinite(d->l2_eps) || !(d->l2_eps >= 0.f) || !std::isfinite(d->scale)) return GDN_EINVAL;
    if (d->n_v_heads % d->n_k_heads != 0) return GDN_ESHAPE;
    if (d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128)) return GDN_ESHAPE;
    if (d->conv_width != 0 && d->conv_width != 4) return GDN_ESHAPE;
    if (d->sub_chunk != GDN_SUB_CHUNK) return GDN_ESHAPE;
    if (d->grid <= 0 || d->grid % GDN_SUB_CHUNK != 0) return GDN_ESHAPE;
    if (n_channels(*d) > (int64_t)1 << 24) return GDN_ESHAPE;
    // a launch must hold at least one sub-chunk of rows (x and o offsets are 32-bit)
    const int64_t row_bytes = std::max<int64_t>(n_channels(*d) * (int64_t)act_size(*d),
                                                (int64_t)d->n_v_heads * d->d_v * (int64_t)out_size(*d));
    if (((int64_t)INT32_MAX - 4 * row_bytes) / row_bytes < kC) return GDN_ESHAPE;
    return GDN_OK;
}

uint64_t gdn_desc_tag(const gdn_desc *d)
{
    if (!d) return 0;
    const int32_t f[8] = {d->n_k_heads, d->n_v_heads, d->d_k,  d->d_v,
                          d->conv_width, d->sub_chunk, d->grid, d->act_dtype};
    uint64_t h = 1469598103934665603ull;  // FNV-1a offset basis
    const unsigned char *p = (const unsigned char *)f;
    for (size_t i = 0; i < sizeof(f); ++i) {
        h ^= p[i];
        h *= 1099511628211ull;  // FNV prime
    }
    return h;
}

size_t gdn_state_S_bytes(const gdn_desc *d)
{
    if (gdn_desc_check(d) != GDN_OK) return 0;
    return (size_t)d->n_v_heads * d->d_k * d->d_v * sizeof(float);
}

size_t gdn_state_conv_bytes(const gdn_desc *d)
{
    if (gdn_desc_check(d) != GDN_OK || d->conv_width == 0) return 0;
    return (size_t)(d->conv_width - 1) * n_channels(*d) * act_size(*d);
}

// Bytes of the scratch final states a branch batch without requested final states writes:
// one S and window per sequence of a launch.
static size_t scratch_states_bytes(const gdn_desc &d, int64_t n_seq)
{
    const size_t one = align256(gdn_state_S_bytes(&d)) + align256(gdn_state_conv_bytes(&d));
    return (size_t)std::min<int64_t>(n_seq, kMaxSegPerLaunch) * one;
}

size_t gdn_workspace_bytes(const gdn_desc *d, int64_t max_rows, int32_t max_segments)
{
    if (gdn_desc_check(d) != GDN_OK || max_rows < 0 || max_segments < 0) return 0;
    return workspace_bytes(*d, max_rows / kC + max_segments) + scratch_states_bytes(*d, max_segments);
}

gdn_status gdn_state_init(const gdn_desc *d, gdn_state *s, void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if ((st = check_dst(*d, s))) return st;
    if (launch_zero(s->S, gdn_state_S_bytes(d), stream) != 0) return GDN_EDEVICE;
    if (d->conv_width > 0 && launch_zero(s->conv, gdn_state_conv_bytes(d), stream) != 0)
        return GDN_EDEVICE;
    s->pos = 0;
    s->tag = gdn_desc_tag(d);
    return GDN_OK;
}

gdn_status gdn_state_capture(const gdn_desc *d, const gdn_state *live, gdn_state *snap,
                             void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if ((st = check_state(*d, live))) return st;
    if ((st = check_dst(*d, snap))) return st;
    if (states_overlap(*d, live, snap)) return GDN_EALIAS;
    if ((st = copy_state(*d, live, snap, stream))) return st;
    snap->pos = live->pos;
    snap->tag = live->tag;
    return GDN_OK;
}

gdn_status gdn_state_restore(const gdn_desc *d, gdn_state *live, const gdn_state *snap,
                             void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if ((st = check_state(*d, snap))) return st;
    if ((st = check_dst(*d, live))) return st;
    if (states_overlap(*d, live, snap)) return GDN_EALIAS;
    if ((st = copy_state(*d, snap, live, stream))) return st;
    live->pos = snap->pos;
    live->tag = snap->tag;
    return GDN_OK;
}

gdn_status gdn_state_fork(const gdn_desc *d, const gdn_state *src, gdn_state *dst, int32_t n,
                          void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if ((st = check_state(*d, src))) return st;
    if (n < 0 || (n > 0 && !dst)) return GDN_EINVAL;
    for (int32_t i = 0; i < n; ++i) {
        if ((st = check_dst(*d, &dst[i]))) return st;
        if (states_overlap(*d, src, &dst[i])) return GDN_EALIAS;
        for (int32_t j = 0; j < i; ++j)
            if (states_overlap(*d, &dst[i], &dst[j])) return GDN_EALIAS;
    }
    for (int32_t i = 0; i < n; ++i) {
        if ((st = copy_state(*d, src, &dst[i], stream))) return st;
        dst[i].pos = src->pos;
        dst[i].tag = src->tag;
    }
    return GDN_OK;
}

gdn_status conv1d_state_step(const gdn_desc *d, const void *x, const void *conv_w, void *window,
                             void *y, int64_t T, void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if (d->conv_width == 0) return GDN_ESHAPE;
    if (T < 0 || T > INT32_MAX) return GDN_EINVAL;
    if (!conv_w || !window || (T > 0 && (!x || !y))) return GDN_EINVAL;
    if (T == 0) return GDN_OK;
    {
        // y and the window are written: neither may overlap x, the weights or each other
        const int64_t C = n_channels(*d);
        const size_t xb = (size_t)(T * C) * act_size(*d), yb = (size_t)(T * C) * out_size(*d);
        const size_t wb = (size_t)C * d->conv_width * act_size(*d);
        const size_t nb = (size_t)(d->conv_width - 1) * C * act_size(*d);
        if (overlap(y, yb, x, xb) || overlap(y, yb, conv_w, wb) || overlap(y, yb, window, nb) ||
            overlap(window, nb, x, xb) || overlap(window, nb, conv_w, wb))
            return GDN_EALIAS;
    }
    // the kernel moves 8 channels per 16-byte (bf16) or two 16-byte (fp32) pieces
    if (!aligned(x, 16) || !aligned(conv_w, 16) || !aligned(window, 16) || !aligned(y, 16))
        return GDN_EINVAL;
    if (launch_conv_step(*d, x, conv_w, window, y, T, stream) != 0) return GDN_EDEVICE;
    return GDN_OK;
}

gdn_status gdn_prefill_chunked(const gdn_desc *d, const void *x, const void *conv_w,
                               const float *g, const float *beta, const gdn_state *in,
                               gdn_state *out, void *o, int64_t T, int32_t mode,
                               int64_t *rows_done, void *ws, size_t ws_bytes, void *stream)
{
    return gdn_prefill_chunked_events(d, x, conv_w, g, beta, in, out, o, T, mode, rows_done, ws,
                                      ws_bytes, stream, nullptr, 0);
}

gdn_status gdn_prefill_chunked_events(const gdn_desc *d, const void *x, const void *conv_w,
                                      const float *g, const float *beta, const gdn_state *in,
                                      gdn_state *out, void *o, int64_t T, int32_t mode,
                                      int64_t *rows_done, void *ws, size_t ws_bytes,
                                      void *stream, void *const *events, int32_t n_events)
{
    if (n_events < 0 || (n_events > 0 && !events)) return GDN_EINVAL;
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if (mode != GDN_COMMIT && mode != GDN_FORK) return GDN_EINVAL;
    if (T < 0 || T > INT32_MAX) return GDN_EINVAL;
    if ((st = check_state(*d, in))) return st;
    if (!out || !out->S || !aligned(out->S, 4)) return GDN_EINVAL;
    if (d->conv_width > 0 && (!out->conv || !aligned(out->conv, 16))) return GDN_EINVAL;
    int64_t n;
    if (mode == GDN_COMMIT) {
        if (in->pos % d->grid != 0) return GDN_EGRID;
        if (!states_same(in, out) && states_overlap(*d, in, out)) return GDN_EALIAS;
        n = (T / d->grid) * d->grid;
    } else {
        if (in->pos % GDN_SUB_CHUNK != 0) return GDN_EGRID;
        if (states_overlap(*d, in, out)) return GDN_EALIAS;
        n = T;
    }
    if (n > 0) {
        if (!x || !g || !beta || !o || (d->conv_width > 0 && !conv_w)) return GDN_EINVAL;
        if (!aligned(x, 16) || !aligned(o, 16) || !aligned(g, 4) || !aligned(beta, 4) ||
            (d->conv_width > 0 && !aligned(conv_w, 16)))
            return GDN_EINVAL;
        const int64_t piece = max_rows_per_launch(*d);
        const size_t ws_used = workspace_bytes(*d, (std::min(n, piece) + kC - 1) / kC);
        if (!ws || ws_bytes < ws_used) return GDN_EWORKSPACE;
        if (!aligned(ws, 16)) return GDN_EINVAL;
        const gdn_state *io_in[1] = {in}, *io_out[1] = {out};
        if (io_overlap(*d, n, x, conv_w, g, beta, o, ws, ws_used, io_in, 1, io_out, 1))
            return GDN_EALIAS;
        const int64_t pos0 = in->pos;
        const uint64_t tag = in->tag;
        for (int64_t r0 = 0; r0 < n; r0 += piece) {
            Seg s;
            std::memset(&s, 0, sizeof(s));
            s.row0 = r0;
            s.n = (int32_t)std::min(piece, n - r0);
            s.S_in = r0 == 0 ? in->S : out->S;
            s.win_in = r0 == 0 ? in->conv : out->conv;
            s.S_out = out->S;
            s.win_out = out->conv;
            std::vector<Seg> segs(1, s);
            if ((st = run_segments(*d, segs, x, conv_w, g, beta, o, ws, stream,
                                   r0 == 0 ? events : nullptr, r0 == 0 ? n_events : 0)))
                return st;
        }
        out->pos = pos0 + n;
        out->tag = tag;
    } else {
        if (!states_same(in, out) && (st = copy_state(*d, in, out, stream))) return st;
        out->pos = in->pos;
        out->tag = in->tag;
    }
    if (rows_done) *rows_done = n;
    return GDN_OK;
}

gdn_status gdn_prefill_branches(const gdn_desc *d, int32_t B, const int64_t *cu_rows,
                                const void *x, const void *conv_w, const float *g,
                                const float *beta, const gdn_state *const *init,
                                gdn_state *const *out, void *o, void *ws, size_t ws_bytes,
                                void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if (B <= 0 || !cu_rows || !init) return GDN_EINVAL;
    if (cu_rows[0] != 0) return GDN_EINVAL;
    for (int32_t b = 0; b < B; ++b) {
        if (cu_rows[b + 1] - cu_rows[b] <= 0) return GDN_EINVAL;  // empty branch
        if (cu_rows[b + 1] - cu_rows[b] > max_rows_per_launch(*d)) return GDN_ESHAPE;
    }
    if (!x || !g || !beta || !o || (d->conv_width > 0 && !conv_w)) return GDN_EINVAL;
    if (!aligned(x, 16) || !aligned(o, 16) || !aligned(g, 4) || !aligned(beta, 4) ||
        (d->conv_width > 0 && !aligned(conv_w, 16)))
        return GDN_EINVAL;
    for (int32_t b = 0; b < B; ++b) {
        if ((st = check_state(*d, init[b]))) return st;
        if (init[b]->pos % GDN_SUB_CHUNK != 0) return GDN_EGRID;
    }
    if (out) {
        for (int32_t b = 0; b < B; ++b) {
            if (!out[b] || !out[b]->S || !aligned(out[b]->S, 4)) return GDN_EINVAL;
            if (d->conv_width > 0 && (!out[b]->conv || !aligned(out[b]->conv, 16))) return GDN_EINVAL;
            for (int32_t j = 0; j < B; ++j)
                if (states_overlap(*d, out[b], init[j])) return GDN_EALIAS;
            for (int32_t j = 0; j < b; ++j)
                if (states_overlap(*d, out[b], out[j])) return GDN_EALIAS;
        }
    }
    std::vector<Seg> segs((size_t)B);
    for (int32_t b = 0; b < B; ++b) {
        Seg &s = segs[b];
        std::memset(&s, 0, sizeof(s));
        s.row0 = cu_rows[b];
        s.n = (int32_t)(cu_rows[b + 1] - cu_rows[b]);
        s.S_in = init[b]->S;
        s.win_in = init[b]->conv;
        // Without requested final states the chain still writes S; it goes to the workspace
        // tail reserved below.
        s.S_out = out ? out[b]->S : nullptr;
        s.win_out = out ? out[b]->conv : nullptr;
    }
    const int64_t subs = max_launch_subs(segs);
    size_t need = workspace_bytes(*d, subs);
    const size_t s_bytes = gdn_state_S_bytes(d), c_bytes = align256(gdn_state_conv_bytes(d));
    if (!out) need += scratch_states_bytes(*d, B);
    if (!ws || ws_bytes < need) return GDN_EWORKSPACE;
    if (!aligned(ws, 16)) return GDN_EINVAL;
    if (io_overlap(*d, cu_rows[B], x, conv_w, g, beta, o, ws, need, init, B,
                   out ? (const gdn_state *const *)out : nullptr, out ? B : 0))
        return GDN_EALIAS;
    if (!out) {
        // scratch final states, reused by every launch group (ordered on the stream)
        char *tail = (char *)ws + workspace_bytes(*d, subs);
        for (int32_t b = 0; b < B; ++b) {
            const int32_t k = b % kMaxSegPerLaunch;
            segs[b].S_out = (float *)(tail + (size_t)k * (align256(s_bytes) + c_bytes));
            segs[b].win_out = d->conv_width > 0 ? tail + (size_t)k * (align256(s_bytes) + c_bytes) +
                                                      align256(s_bytes)
                                                : nullptr;
        }
    }
    std::vector<int64_t> pos0((size_t)B);
    for (int32_t b = 0; b < B; ++b) pos0[b] = init[b]->pos;
    const uint64_t tag = gdn_desc_tag(d);
    if ((st = run_segments(*d, segs, x, conv_w, g, beta, o, ws, stream))) return st;
    if (out)
        for (int32_t b = 0; b < B; ++b) {
            out[b]->pos = pos0[b] + (cu_rows[b + 1] - cu_rows[b]);
            out[b]->tag = tag;
        }
    return GDN_OK;
}

gdn_status gdn_decode_step(const gdn_desc *d, int32_t B, const void *x, const void *conv_w,
                           const float *g, const float *beta, const gdn_state *const *in,
                           gdn_state *const *out, void *o, void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if (B <= 0 || !in || !out || !x || !g || !beta || !o || (d->conv_width > 0 && !conv_w))
        return GDN_EINVAL;
    if (!aligned(x, 16) || !aligned(o, 16) || !aligned(g, 4) || !aligned(beta, 4) ||
        (d->conv_width > 0 && !aligned(conv_w, 16)))
        return GDN_EINVAL;
    for (int32_t b = 0; b < B; ++b) {
        if ((st = check_state(*d, in[b]))) return st;
        // the step moves S in 16-byte pieces
        if (!aligned(in[b]->S, 16)) return GDN_EINVAL;
        if (!out[b] || !out[b]->S || !aligned(out[b]->S, 16)) return GDN_EINVAL;
        if (d->conv_width > 0 && (!out[b]->conv || !aligned(out[b]->conv, 16))) return GDN_EINVAL;
    }
    // out[b] is in[b] itself or disjoint from it, and disjoint from every other sequence's
    // states: each workgroup reads and rewrites only its own sequence's tiles.
    for (int32_t b = 0; b < B; ++b) {
        if (!states_same(in[b], out[b]) && states_overlap(*d, in[b], out[b])) return GDN_EALIAS;
        for (int32_t j = 0; j < B; ++j) {
            if (j == b) continue;
            if (states_overlap(*d, out[b], in[j])) return GDN_EALIAS;
            if (j < b && states_overlap(*d, out[b], out[j])) return GDN_EALIAS;
        }
    }
    // o may overlap no input and no state; no final state may overlap an input
    if (io_overlap(*d, B, x, conv_w, g, beta, o, nullptr, 0, in, B, (const gdn_state *const *)out, B))
        return GDN_EALIAS;
    std::vector<int64_t> pos0((size_t)B);
    for (int32_t b = 0; b < B; ++b) pos0[b] = in[b]->pos;
    const uint64_t tag = gdn_desc_tag(d);
    const int64_t C = n_channels(*d);
    const size_t xb = (size_t)C * act_size(*d), ob = (size_t)d->n_v_heads * d->d_v * out_size(*d);
    for (int32_t b0 = 0; b0 < B; b0 += kMaxSegPerLaunch) {
        const int32_t n = std::min<int32_t>(kMaxSegPerLaunch, B - b0);
        DecodeArgs da;
        SegArgs wa;
        std::memset(&da, 0, sizeof(da));
        std::memset(&wa, 0, sizeof(wa));
        for (int32_t i = 0; i < n; ++i) {
            const int32_t b = b0 + i;
            DecodeSeq &q = da.seq[i];
            q.x = (const char *)x + (size_t)b * xb;
            q.S_in = in[b]->S;
            q.S_out = out[b]->S;
            q.win = in[b]->conv;
            // a window other than the one read is written by the step itself
            const bool sep = d->conv_width > 0 &&
                             !overlap(in[b]->conv, gdn_state_conv_bytes(d), out[b]->conv,
                                      gdn_state_conv_bytes(d));
            q.win_out = sep ? out[b]->conv : nullptr;
            q.g = g + (size_t)b * d->n_v_heads;
            q.beta = beta + (size_t)b * d->n_v_heads;
            q.o = (char *)o + (size_t)b * ob;
            if (d->conv_width > 0 && !sep) {  // in-place window: shifted by a second kernel
                Seg &w = wa.seg[wa.n_seg++];
                w.row0 = b;  // row b of x
                w.n = 1;
                w.win_in = in[b]->conv;
                w.win_out = out[b]->conv;
            }
        }
        da.n = n;
        if (launch_decode(*d, da, wa, x, conv_w, stream) != 0) return GDN_EDEVICE;
    }
    for (int32_t b = 0; b < B; ++b) {
        out[b]->pos = pos0[b] + 1;
        out[b]->tag = tag;
    }
    return GDN_OK;
}

size_t gdn_state_file_header_bytes(void) { return sizeof(StateFileHeader); }

gdn_status gdn_state_file_write(const gdn_desc *d, const void *S_host, const void *conv_host,
                                int64_t pos, uint64_t weights_hash, const char *path)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if (!S_host || (d->conv_width > 0 && !conv_host) || !path || !*path || pos < 0)
        return GDN_EINVAL;
    return write_state_file(*d, S_host, conv_host, pos, weights_hash, path);
}

gdn_status gdn_state_file_read(const gdn_desc *d, void *S_host, void *conv_host, int64_t *pos,
                               uint64_t weights_hash, const char *path)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if (!S_host || (d->conv_width > 0 && !conv_host) || !pos || !path || !*path) return GDN_EINVAL;
    return read_state_file(*d, S_host, conv_host, pos, weights_hash, path);
}

gdn_status gdn_state_save(const gdn_desc *d, const gdn_state *state, uint64_t weights_hash,
                          const char *path, void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if ((st = check_state(*d, state))) return st;
    if (!path || !*path) return GDN_EINVAL;
    const size_t sb = gdn_state_S_bytes(d), cb = gdn_state_conv_bytes(d);
    std::vector<unsigned char> host(sb + cb);
    if (copy_to_host(host.data(), state->S, sb, stream) != 0 ||
        (cb && copy_to_host(host.data() + sb, state->conv, cb, stream) != 0) || stream_sync(stream) != 0)
        return GDN_EDEVICE;
    return write_state_file(*d, host.data(), host.data() + sb, state->pos, weights_hash, path);
}

gdn_status gdn_state_load(const gdn_desc *d, gdn_state *state, uint64_t weights_hash,
                          const char *path, void *stream)
{
    gdn_status st = gdn_desc_check(d);
    if (st) return st;
    if (!state || !state->S || !aligned(state->S, 4)) return GDN_EINVAL;
    if (d->conv_width > 0 && (!state->conv || !aligned(state->conv, 16))) return GDN_EINVAL;
    if (!path || !*path) return GDN_EINVAL;
    const size_t sb = gdn_state_S_bytes(d), cb = gdn_state_conv_bytes(d);
    std::vector<unsigned char> host(sb + cb);
    int64_t pos = 0;
    if ((st = read_state_file(*d, host.data(), host.data() + sb, &pos, weights_hash, path))) return st;
    if (copy_to_device(state->S, host.data(), sb, stream) != 0 ||
        (cb && copy_to_device(state->conv, host.data() + sb, cb, stream) != 0) || stream_sync(stream) != 0)
        return GDN_EDEVICE;
    state->pos = pos;
    state->tag = gdn_desc_tag(d);
    return GDN_OK;
}

gdn_status gdn_linear(int64_t T, int32_t K, int32_t N, const void *x, const void *w, void *y,
                      int32_t out_dtype, void *stream)
{
    if (T < 0 || K <= 0 || N <= 0 || K % 64 != 0 || N % 16 != 0) return GDN_EINVAL;
    if (out_dtype != GDN_BF16 && out_dtype != GDN_F32) return GDN_EINVAL;
    if (T > (int64_t)INT32_MAX * 128) return GDN_EINVAL;
    if (T == 0) return GDN_OK;
    if (!x || !w || !y || !aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return GDN_EINVAL;
    const size_t yb = (size_t)T * N * (out_dtype == GDN_BF16 ? 2 : 4);
    if (overlap(y, yb, x, (size_t)T * K * 2) || overlap(y, yb, w, (size_t)N * K * 2)) return GDN_EALIAS;
    if (launch_linear(T, K, N, x, w, y, out_dtype, stream) != 0) return GDN_EDEVICE;
    return GDN_OK;
}

static bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

gdn_status gdn_attention_prefill(const gdn_attn_desc *desc, int32_t B, const gdn_attn_seq *seqs,
                                 void *stream)
{
    if (!desc || B < 0 || (B > 0 && !seqs)) return GDN_EINVAL;
    const gdn_attn_desc &d = *desc;
    if (d.out_dtype != GDN_BF16 && d.out_dtype != GDN_F32) return GDN_EINVAL;
    if (!(d.scale > 0.f) || !std::isfinite(d.scale)) return GDN_EINVAL;
    if (d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.n_q_heads % d.n_kv_heads != 0) return GDN_ESHAPE;
    const int R = d.n_q_heads / d.n_kv_heads;
    if (!(R == 1 || R == 2 || R == 4 || R % 8 == 0)) return GDN_ESHAPE;
    if (d.head_dim != 128 && d.head_dim != 256) return GDN_ESHAPE;
    const int HW = attn_heads_per_wg(d.n_q_heads, d.n_kv_heads);
    const int64_t rows_per_tile = 16 * (8 / HW);
    const int64_t n_groups = (int64_t)d.n_kv_heads * (R / HW);
    const size_t out_el = d.out_dtype == GDN_BF16 ? 2 : 4;
    const int64_t qrow = (int64_t)d.n_q_heads * d.head_dim, kvrow = (int64_t)d.n_kv_heads * d.head_dim;
    for (int32_t i = 0; i < B; ++i) {
        const gdn_attn_seq &q = seqs[i];
        if (q.T < 0 || q.pos0 < 0 || q.T > ((int64_t)1 << 40) || q.pos0 > ((int64_t)1 << 40))
            return GDN_EINVAL;
        if (q.T == 0) continue;
        if (!q.q || !q.k || !q.v || !q.o) return GDN_EINVAL;
        if (!aligned(q.q, 16) || !aligned(q.k, 16) || !aligned(q.v, 16) || !aligned(q.o, 16))
            return GDN_EINVAL;
        if (((q.T + rows_per_tile - 1) / rows_per_tile) * n_groups > INT32_MAX) return GDN_EINVAL;
        const size_t ob = (size_t)(q.T * qrow) * out_el, qb = (size_t)(q.T * qrow) * 2;
        const size_t kb = (size_t)((q.pos0 + q.T) * kvrow) * 2;
        if (ranges_overlap(q.o, ob, q.q, qb) || ranges_overlap(q.o, ob, q.k, kb) ||
            ranges_overlap(q.o, ob, q.v, kb))
            return GDN_EALIAS;
    }
    const float c2 = d.scale * 1.4426950408889634f;  // scores in units of log2
    AttnArgs aa;
    aa.n = 0;
    int64_t tiles = 0;
    auto flush = [&]() -> int {
        if (aa.n == 0) return 0;
        const int r = launch_attention(aa, (int)tiles, d.n_q_heads, d.n_kv_heads, d.head_dim, HW,
                                       c2, d.out_dtype, stream);
        aa.n = 0;
        tiles = 0;
        return r;
    };
    for (int32_t i = 0; i < B; ++i) {
        const gdn_attn_seq &q = seqs[i];
        if (q.T == 0) continue;
        const int64_t nt = (q.T + rows_per_tile - 1) / rows_per_tile;
        if (aa.n == kMaxSegPerLaunch || (tiles + nt) * n_groups > INT32_MAX)
            if (flush() != 0) return GDN_EDEVICE;
        AttnSeq &s = aa.seq[aa.n++];
        s.q = q.q;
        s.k = q.k;
        s.v = q.v;
        s.o = q.o;
        s.pos0 = q.pos0;
        s.T = q.T;
        s.tile0 = (int32_t)tiles;
        tiles += nt;
    }
    if (flush() != 0) return GDN_EDEVICE;
    return GDN_OK;
}

int64_t gdn_commit_rows(int64_t n, int32_t grid)
{
    if (n < 0 || grid <= 0) return -1;
    return (n / grid) * grid;
}

int64_t gdn_shared_prefix_rows(int64_t state_pos, int64_t prefix_end)
{
    if (state_pos < 0 || state_pos % GDN_SUB_CHUNK != 0 || prefix_end < state_pos) return -1;
    const int64_t end = (prefix_end / GDN_SUB_CHUNK) * GDN_SUB_CHUNK;
    return end > state_pos ? end - state_pos : 0;
}

gdn_status gdn_ckpt_init(gdn_ckpt_ring *r, int32_t cap)
{
    if (!r || cap <= 0 || cap > GDN_MAX_CHECKPOINTS) return GDN_EINVAL;
    std::memset(r, 0, sizeof(*r));
    r->cap = cap;
    for (int i = 0; i < GDN_MAX_CHECKPOINTS; ++i) r->pos[i] = -1;
    return GDN_OK;
}

int32_t gdn_ckpt_push(gdn_ckpt_ring *r, int64_t pos)
{
    if (!r || r->cap <= 0 || r->cap > GDN_MAX_CHECKPOINTS || pos < 0) return -1;
    int32_t slot = -1;
    for (int32_t i = 0; i < r->cap && slot < 0; ++i)
        if (r->pos[i] == pos) slot = i;
    for (int32_t i = 0; i < r->cap && slot < 0; ++i)
        if (r->pos[i] < 0) slot = i;
    if (slot < 0) {  // evict the oldest
        slot = 0;
        for (int32_t i = 1; i < r->cap; ++i)
            if (r->age[i] < r->age[slot]) slot = i;
    }
    if (r->pos[slot] < 0) r->n++;
    r->pos[slot] = pos;
    r->age[slot] = ++r->clock;
    return slot;
}

int32_t gdn_ckpt_find(const gdn_ckpt_ring *r, int64_t d)
{
    if (!r || r->cap <= 0 || r->cap > GDN_MAX_CHECKPOINTS) return -1;
    int32_t best = -1;
    for (int32_t i = 0; i < r->cap; ++i)
        if (r->pos[i] >= 0 && r->pos[i] <= d && (best < 0 || r->pos[i] > r->pos[best])) best = i;
    return best;
}

int32_t gdn_ckpt_drop_above(gdn_ckpt_ring *r, int64_t d)
{
    if (!r || r->cap <= 0 || r->cap > GDN_MAX_CHECKPOINTS) return 0;
    int32_t n = 0;
    for (int32_t i = 0; i < r->cap; ++i)
        if (r->pos[i] >= 0 && r->pos[i] > d) {  // live slots only (empty ones hold -1)
            r->pos[i] = -1;
            r->age[i] = 0;
            r->n--;
            n++;
        }
    return n;
}

const char *gdn_status_str(gdn_status s)
{
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument";
    case GDN_ESHAPE: return "unsupported shape";
    case GDN_EGRID: return "start position not on the required grid";
    case GDN_EMISMATCH: return "state tag does not match the descriptor";
    case GDN_EWORKSPACE: return "workspace missing or too small";
    case GDN_EDEVICE: return "HIP launch or copy failed";
    case GDN_EALIAS: return "output state overlaps memory it must not";
    case GDN_EFILE: return "state file missing, unreadable, truncated, corrupt or not writable";
    default: return "unknown status";
    }
}

}  // extern "C"
