// gdn_backend_host.cpp -- test stand-in for the device half of libgdn_prefill.so.
//
// Linked with csrc/gdn_host.cpp (the library's whole host half, unchanged) into
// libgdn_hostcheck.so, which the CPU tests load instead of the HIP library.  "Device" pointers
// are host memory here: zero, copy and the host <-> device copies are memset / memcpy, so the
// state operations, state files and the session store run for real on host buffers.  The
// kernel launchers compute nothing: each records what it was asked to launch (the sequences
// of a prefill launch with their rows, sub-chunks and states), which the tests read back to
// check the launch plan.  Built with g++ (optionally with AddressSanitizer and
// UndefinedBehaviorSanitizer); includes no ROCm header.
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../hybrid_linear_attention_prefill_amd/csrc/gdn_internal.h"

namespace {

enum Kind { kPrefill = 1, kDecode = 2, kConv = 3, kLinear = 4, kAttention = 5 };

struct Record {
    int kind;
    int64_t rows;  // prefill: sub-chunks of the launch; decode: sequences; others: rows / T
    std::vector<gdn::Seg> segs;
};

std::mutex g_mu;
std::vector<Record> g_log;

void record(int kind, int64_t rows, const gdn::SegArgs *sa)
{
    std::lock_guard<std::mutex> lk(g_mu);
    Record r;
    r.kind = kind;
    r.rows = rows;
    if (sa)
        for (int i = 0; i < sa->n_seg; ++i) r.segs.push_back(sa->seg[i]);
    g_log.push_back(r);
}

}  // namespace

namespace gdn {

int launch_prefill(const gdn_desc &, const SegArgs &sa, const void *, const void *, const float *,
                   const float *, void *, const Workspace &, void *, void *const *, int)
{
    record(kPrefill, sa.n_sub, &sa);
    return 0;
}

int launch_decode(const gdn_desc &, const DecodeArgs &da, const SegArgs &, const void *,
                  const void *, void *)
{
    record(kDecode, da.n, nullptr);
    return 0;
}

int launch_conv_step(const gdn_desc &, const void *, const void *, void *, void *, int64_t T, void *)
{
    record(kConv, T, nullptr);
    return 0;
}

int launch_linear(int64_t T, int, int, const void *, const void *, void *, int, void *)
{
    record(kLinear, T, nullptr);
    return 0;
}

int launch_attention(const AttnArgs &aa, int, int, int, int, int, float, int, void *)
{
    record(kAttention, aa.n, nullptr);
    return 0;
}

int launch_zero(void *p, size_t bytes, void *)
{
    std::memset(p, 0, bytes);
    return 0;
}

int launch_copy(void *dst, const void *src, size_t bytes, void *)
{
    std::memmove(dst, src, bytes);
    return 0;
}

int copy_to_host(void *host, const void *dev, size_t bytes, void *)
{
    std::memcpy(host, dev, bytes);
    return 0;
}

int copy_to_device(void *dev, const void *host, size_t bytes, void *)
{
    std::memcpy(dev, host, bytes);
    return 0;
}

int stream_sync(void *) { return 0; }

}  // namespace gdn

extern "C" {

// Number of kernel launches recorded since the last reset.
int32_t gdn_hostcheck_launches(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    return (int32_t)g_log.size();
}

void gdn_hostcheck_reset(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    g_log.clear();
}

// Launch i: returns its kind (1 prefill, 2 decode, 3 conv, 4 linear, 5 attention) and writes
// its size (sub-chunks, sequences or rows) to *rows and its sequence count to *n_seg; with
// `segs` non-null, up to max_segs sequences as 7 int64 each: row0, n, sub0, S_in, win_in,
// S_out, win_out.  -1 when i is out of range.
int32_t gdn_hostcheck_launch(int32_t i, int64_t *rows, int32_t *n_seg, int64_t *segs,
                             int32_t max_segs)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (i < 0 || (size_t)i >= g_log.size()) return -1;
    const Record &r = g_log[(size_t)i];
    if (rows) *rows = r.rows;
    if (n_seg) *n_seg = (int32_t)r.segs.size();
    for (int k = 0; segs && k < max_segs && (size_t)k < r.segs.size(); ++k) {
        const gdn::Seg &s = r.segs[(size_t)k];
        int64_t *o = segs + 7 * k;
        o[0] = s.row0;
        o[1] = s.n;
        o[2] = s.sub0;
        o[3] = (int64_t)(intptr_t)s.S_in;
        o[4] = (int64_t)(intptr_t)s.win_in;
        o[5] = (int64_t)(intptr_t)s.S_out;
        o[6] = (int64_t)(intptr_t)s.win_out;
    }
    return r.kind;
}

}  // extern "C"
