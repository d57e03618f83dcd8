/*
 * gdn.h -- C ABI of libgdn_prefill.so: chunked prefill of one Gated DeltaNet layer on an
 * AMD Instinct MI355X (gfx950), with a recurrent state that is carried across calls,
 * committed only on a fixed absolute-position grid, captured, restored and forked.
 *
 * Sources of the behaviour (page title, section):
 *  - "The shadow reader", section "Exact on a grid": the state advances only in whole grid
 *    chunks at absolute positions k*grid; the rows past the last grid line wait as a
 *    pending tail; a question runs the tail plus its own rows above the committed rows and
 *    the state is put back afterwards (a fork); replay equals a fresh prefill bit for bit.
 *  - "The shadow reader", sections "One session's state" and "Exact on a grid": up to six
 *    checkpoints, one per turn's prompt end; on a differing prompt go back to the newest
 *    checkpoint at or below the first differing token, or start over.
 *  - PR "qwen3_5: run prompts that share prefixes once per prefix", section Purpose: a
 *    prefix state holds the fp32 recurrent state and the three most recent conv inputs; each
 *    prefix is run up to its last multiple of 64 rows and the remainder runs with every
 *    later group or branch; each branch continues from the shared state; invalid requests
 *    are refused before any device work (section "Test Result").
 *  - "Long context and sessions", section "Sessions on one engine": states are exported,
 *    imported and copied between slots; a state made for another layer shape is refused.
 *
 * Conventions for every call below:
 *  - Pointers named "device" point to GPU memory owned by the caller; the library allocates
 *    no device memory and keeps no pointer after a call returns.  Host pointers likewise.
 *  - Every argument is validated on the host first.  A negative return means nothing was
 *    enqueued and no state byte, position or tag changed.
 *  - Device pointers must be aligned: 16 bytes for x, conv_w, o, conv windows and the
 *    workspace, 4 bytes for g, beta and S (GDN_EINVAL otherwise).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *    returns without synchronising.  GDN_EDEVICE reports a failed launch or copy; the
 *    outputs are then undefined.
 *  - The library holds no global mutable state (gdn_prefill_chunked_noalloc's static
 *    workspace aside); calls on different streams may overlap as long as they write disjoint
 *    memory (and use different workspaces).  GDN_TEST_LAUNCH_ROWS in the environment (a
 *    positive multiple of 64) lowers the rows a prefill launch takes, for tests of the
 *    chained-launch path; it never raises them.
 *  - Admissible magnitudes.  The prefill's matrix products take fp16 operands (11-bit
 *    significand, range 6.1e-5 .. 65504) with fp32 accumulation: the normalised q and k, the
 *    factors Tinv and M (|entries| <= 1 in practice), and, scaled with the values, an fp16 copy
 *    of the state S, R = beta v - beta gamma K S and D = Tinv R.  Outputs and states match the
 *    float64 per-token rule to 2e-3 relative L2 while the largest |S| entry and the largest
 *    post-conv |v| of a call stay within about 1e-4 .. 2e4 (measured on the 16/32/128 layer:
 *    max |S| from 1.3e-4 to 2.4e4 passes; at 8e-6, fp16 subnormals give 9e-3; at 4.7e4 an fp16
 *    operand overflows and the outputs are not finite).  The state itself, the gates, conv and
 *    norms are fp32 throughout.
 *
 * Layouts (row-major, innermost last):
 *   C   = 2*n_k_heads*d_k + n_v_heads*d_v conv channels, ordered q | k | v, each head's
 *         dims contiguous; value head h reads key head h / (n_v_heads / n_k_heads).
 *   x   [T][C]          act dtype  pre-conv inputs (post-conv when conv_width == 0)
 *   conv_w [C][W]       act dtype  tap W-1 multiplies the current row
 *   g, beta [T][Hv]     fp32       g <= 0 (log decay), beta in (0,1) (write strength)
 *   o   [T][Hv][d_v]    out dtype
 *   S   [Hv][d_k][d_v]  fp32       recurrent state
 *   conv window [W-1][C] act dtype, oldest row first (the last W-1 conv inputs)
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gdn_status;
enum {
    GDN_OK = 0,
    GDN_EINVAL = -1,     /* null pointer, bad enum value, negative or empty size */
    GDN_ESHAPE = -2,     /* head counts / dims / conv width / sub-chunk not supported */
    GDN_EGRID = -3,      /* a start position is not on the grid the mode requires */
    GDN_EMISMATCH = -4,  /* a state's tag is not the descriptor's tag */
    GDN_EWORKSPACE = -5, /* workspace missing or smaller than gdn_workspace_bytes() */
    GDN_EDEVICE = -6,    /* a HIP launch or copy failed */
    GDN_EALIAS = -7,     /* an output (state, o or workspace) overlaps memory it must not */
    GDN_EFILE = -8,      /* a state file is missing, unreadable, truncated or corrupt, or
                            cannot be written */
};

enum { GDN_F32 = 0, GDN_BF16 = 1 };  /* element types of x / conv / window and of o */
enum { GDN_COMMIT = 0, GDN_FORK = 1 };

#define GDN_SUB_CHUNK 64 /* the only arithmetic boundary of the chunked form */
#define GDN_MAX_CHECKPOINTS 6

/* Layer description.  Supported by the kernels: d_k == d_v in {64, 128};
 * n_v_heads % n_k_heads == 0; conv_width in {0, 4}; sub_chunk == 64;
 * grid a positive multiple of 64 (512 by default).  scale is the output scale
 * (d_k^-1/2 usually; finite); l2_eps (finite, >= 0) sits inside the square root of the q/k
 * normalisation. */
typedef struct {
    int32_t n_k_heads, n_v_heads, d_k, d_v;
    int32_t conv_width; /* 4, or 0 = inputs already post-conv */
    int32_t sub_chunk;  /* must be 64 */
    int32_t grid;       /* commit grid in rows */
    int32_t act_dtype;  /* GDN_BF16 or GDN_F32 */
    int32_t out_dtype;  /* GDN_BF16 or GDN_F32 */
    int32_t conv_silu;  /* 0 = plain conv, 1 = SiLU after the conv */
    float scale;
    float l2_eps;
} gdn_desc;

/* One recurrent state.  S and conv are device pointers owned by the caller
 * (conv may be NULL when conv_width == 0).  pos = absolute rows absorbed; tag identifies
 * the descriptor the state was made for (gdn_desc_tag). */
typedef struct {
    float *S;
    void *conv;
    int64_t pos;
    uint64_t tag;
} gdn_state;

/* ---------------------------------------------------------------- sizes and identity */

/* 0 if the descriptor is supported, else GDN_EINVAL / GDN_ESHAPE. */
gdn_status gdn_desc_check(const gdn_desc *desc);

/* Tag of a descriptor: a 64-bit FNV-1a hash of the fields that fix a state's meaning
 * (heads, dims, conv width, sub-chunk, grid, act dtype).  A state is refused by
 * gdn_state_restore and the prefill calls when its tag differs ("Long context and
 * sessions", section "Sessions on one engine"; "The shadow reader", section
 * "Memory and the disk": another grid does not read it). */
uint64_t gdn_desc_tag(const gdn_desc *desc);

/* Bytes of S ([Hv][d_k][d_v] fp32) and of the conv window ([W-1][C] act dtype). */
size_t gdn_state_S_bytes(const gdn_desc *desc);
size_t gdn_state_conv_bytes(const gdn_desc *desc);

/* Device workspace needed by a prefill call of at most max_rows rows in total over at most
 * max_segments sequences (1 for gdn_prefill_chunked, B for gdn_prefill_branches; with B it also
 * covers the scratch final states of a branch batch given no output states).
 * 0 on an invalid descriptor. */
size_t gdn_workspace_bytes(const gdn_desc *desc, int64_t max_rows, int32_t max_segments);

/* ---------------------------------------------------------------- state operations */

/* Zero S and the window on `stream`; pos = 0; tag = gdn_desc_tag(desc).  The state a session
 * starts from, and the one a restore falls back to when no checkpoint lies at or below the
 * first differing token ("The shadow reader", section "Exact on a grid").  Refuses a
 * destination whose S is not 4-byte or whose window is not 16-byte aligned (GDN_EINVAL). */
gdn_status gdn_state_init(const gdn_desc *desc, gdn_state *state, void *stream);

/* snap <- live: device copies of S and the window plus pos and tag ("Long context and
 * sessions", section "Sessions on one engine": a session's state is saved into a slot as a GPU
 * copy; "The shadow reader", section "One session's state": a checkpoint of the recurrent state
 * at a turn's end).  Refuses a live state of another tag (GDN_EMISMATCH), snap == live or
 * overlapping buffers (GDN_EALIAS) and a misaligned snap (GDN_EINVAL). */
gdn_status gdn_state_capture(const gdn_desc *desc, const gdn_state *live, gdn_state *snap,
                             void *stream);

/* live <- snap ("Long context and sessions", section "Sessions on one engine": a slot is loaded
 * back exactly, and a state made for other layers is refused; "The shadow reader", section
 * "Exact on a grid": on a differing prompt the newest checkpoint at or below the first
 * differing token is restored).  Refuses a snapshot whose tag is not the descriptor's
 * (GDN_EMISMATCH): a state for another layer shape or grid is not read. */
gdn_status gdn_state_restore(const gdn_desc *desc, gdn_state *live, const gdn_state *snap,
                             void *stream);

/* dst[i] <- src for i in [0, n): n device copies (slots for a batch of branches, or the scratch
 * state a question runs in while the committed state stays as it was: "The shadow reader",
 * section "Exact on a grid"; PR "qwen3_5: run prompts that share prefixes once per prefix",
 * section Purpose: every branch continues from a copy of the shared prefix state). */
gdn_status gdn_state_fork(const gdn_desc *desc, const gdn_state *src, gdn_state *dst, int32_t n,
                          void *stream);

/* ---------------------------------------------------------------- state files */

/* A state file holds one state (S, the conv window, pos) with a header that records the
 * layer descriptor's fields and tag (heads, dims, conv width, sub-chunk, grid, act dtype) and a
 * caller-chosen 64-bit hash of the model weights.  A file for another layer shape, grid,
 * dtype or weights is refused (GDN_EMISMATCH) and the state is left as it was; a missing,
 * short or corrupt file (FNV-1a checksums over header and payload) gives GDN_EFILE ("The
 * shadow reader", sections "Memory and the disk" and "Memory": a session goes to disk and
 * comes back exact, and a file for another model or grid is not read; "Long context and
 * sessions", section "On disk, across reloads": a copy for other layers reads as missing,
 * and a failed write leaves the slot missing, never stale).
 *
 * Writing first removes any file at `path`, then writes `path`.tmp.<pid>, flushes it to disk
 * and renames it to `path`: a failed or interrupted write leaves no file at `path`.
 * Layout (little-endian): a 104-byte header {char[8] "GDNSTAT1", u32 version = 1,
 * u32 header bytes = 104, i32 n_k_heads, n_v_heads, d_k, d_v, conv_width, sub_chunk, grid,
 * act_dtype, u64 tag, u64 weights_hash, i64 pos, u64 S bytes, u64 window bytes,
 * u64 FNV-1a of the payload, u64 FNV-1a of the preceding 96 header bytes}, then S, then the
 * window. */
size_t gdn_state_file_header_bytes(void);

/* Host-buffer forms: S_host [Hv][d_k][d_v] fp32 and conv_host [W-1][C] act dtype are host
 * memory (conv_host may be NULL when conv_width == 0). */
gdn_status gdn_state_file_write(const gdn_desc *desc, const void *S_host, const void *conv_host,
                                int64_t pos, uint64_t weights_hash, const char *path);
/* Reads and verifies the whole file before writing S_host, conv_host and *pos. */
gdn_status gdn_state_file_read(const gdn_desc *desc, void *S_host, void *conv_host, int64_t *pos,
                               uint64_t weights_hash, const char *path);

/* Device forms: copy the state through host memory.  Both synchronise `stream` (work queued
 * on it that writes the state completes first; a load's copy completes before returning).
 * gdn_state_save refuses a state of another tag (GDN_EMISMATCH); gdn_state_load sets pos and
 * tag only after the copy succeeded. */
gdn_status gdn_state_save(const gdn_desc *desc, const gdn_state *state, uint64_t weights_hash,
                          const char *path, void *stream);
gdn_status gdn_state_load(const gdn_desc *desc, gdn_state *state, uint64_t weights_hash,
                          const char *path, void *stream);

/* ---------------------------------------------------------------- session store */

/* Many sessions over a few device state slots under a byte cap ("The shadow reader", section
 * "Memory and the disk": resident states are capped; past the cap the least recently used
 * session goes to disk, one file a session, and comes back exact when it is fed again; without
 * a disk it is dropped and read again from the start; a planned stop writes every resident
 * session; a file for other weights or another grid is not read.  "Long context and
 * sessions", section "Sessions on one engine": a session comes back from a GPU slot, from disk
 * or fresh, and past the number of GPU slots the least recently used ones leave).
 *
 * The caller owns all memory: n_slots device states (S and window buffers) and a table of
 * max_entries (>= n_slots) entries, one per known session.  At most max_resident =
 * min(n_slots, cap_bytes / (S bytes + window bytes)) sessions are resident at once.  Files
 * are <dir>/gdn-<id as 16 hex digits>.state in the state-file format above (written by
 * gdn_state_save, so a failed write leaves no file).  Host calls; the device work (state
 * copies, zeroing) runs on `stream` and is synchronised where a file is written or read.
 * Not thread-safe: one caller at a time per store. */
enum { GDN_STORE_UNUSED = 0, GDN_STORE_RESIDENT = 1, GDN_STORE_ON_DISK = 2, GDN_STORE_DROPPED = 3 };
enum { GDN_STORE_WAS_RESIDENT = 0, GDN_STORE_FROM_DISK = 1, GDN_STORE_FRESH = 2 };

typedef struct {
    uint64_t id;       /* the caller's session id */
    int64_t pos;       /* the session's position when it last left or entered a slot */
    uint64_t last_use; /* store clock at its last acquire (least recently used = smallest) */
    int32_t slot;      /* device slot while resident, else -1 */
    int32_t where;     /* GDN_STORE_UNUSED / RESIDENT / ON_DISK / DROPPED */
} gdn_store_entry;

typedef struct {
    gdn_desc desc;
    gdn_state *slots;         /* [n_slots] the caller's device states */
    int32_t n_slots, max_resident;
    size_t cap_bytes, state_bytes;
    gdn_store_entry *entries; /* [max_entries] the caller's table */
    int32_t max_entries, reserved;
    uint64_t weights_hash, clock;
    char dir[512];            /* spill directory; "" = no disk (evicted sessions are dropped) */
} gdn_store;

/* Sets up a store over the caller's slots and entry table; dir may be NULL (no disk).
 * GDN_EINVAL when the cap holds no state, max_entries < n_slots, a slot lacks a buffer or dir
 * is too long. */
gdn_status gdn_store_init(gdn_store *store, const gdn_desc *desc, gdn_state *slots,
                          int32_t n_slots, size_t cap_bytes, const char *dir,
                          uint64_t weights_hash, gdn_store_entry *entries, int32_t max_entries);
/* Makes session `id` resident and most recently used; *state points at its slot, which the
 * caller then prefills in place (commits move its pos).  *origin: GDN_STORE_WAS_RESIDENT, or
 * GDN_STORE_FROM_DISK (read back exactly from its file), or GDN_STORE_FRESH (a zero state at
 * pos 0: a new session, one dropped without a disk, or one whose file was missing, damaged or
 * made for other weights or grid; the caller reads it again from the start).  When no slot is
 * free the least recently used resident session is written to its file (or dropped). */
gdn_status gdn_store_acquire(gdn_store *store, uint64_t id, gdn_state **state, int32_t *origin,
                             void *stream);
/* Moves a resident session out of its slot now (to disk, or dropped without one). */
gdn_status gdn_store_evict(gdn_store *store, uint64_t id, void *stream);
/* Writes every resident session to its file; they stay resident (a planned stop). */
gdn_status gdn_store_flush(gdn_store *store, void *stream);
/* Forgets a session and removes its file. */
gdn_status gdn_store_drop(gdn_store *store, uint64_t id);
/* Index of session id in the entry table, or -1. */
int32_t gdn_store_find(const gdn_store *store, uint64_t id);

/* ---------------------------------------------------------------- compute */

/* Standalone causal depthwise conv over all C channels with the window carried (PR "qwen3_5:
 * run prompts that share prefixes once per prefix", section Purpose: the state of a linear-
 * attention layer holds the three most recent conv inputs, which a continuation needs):
 * xt = window ++ x; y[t][c] = sum_j conv_w[c][j] * xt[t+j][c] (SiLU if desc->conv_silu);
 * the window becomes the last W-1 rows of xt.  y [T][C] in desc->out_dtype (device),
 * x [T][C] act dtype (device), window [W-1][C] act dtype (device, updated in place).
 * T >= 0; requires conv_width > 0.  x, conv_w, window and y must be 16-byte aligned
 * (GDN_EINVAL).  y and the window may overlap neither x, conv_w nor each other (GDN_EALIAS). */
gdn_status conv1d_state_step(const gdn_desc *desc, const void *x, const void *conv_w, void *window,
                             void *y, int64_t T, void *stream);

/* Prefill T rows of one sequence from state `in` into state `out`, writing o ("The shadow
 * reader", section "Exact on a grid": the state advances in whole grid chunks at absolute
 * positions; the rows past the last grid line wait as the pending tail; a question runs the
 * tail plus its own rows from the committed state in a fork that leaves that state as it was;
 * a replay equals a fresh prefill bit for bit).
 *
 * GDN_COMMIT: requires in->pos % grid == 0.  Absorbs rows_done = floor(T / grid) * grid
 *   rows (the rest is the caller's pending tail) and writes o rows [0, rows_done).
 *   out may equal in (in-place commit); out->pos = in->pos + rows_done.
 * GDN_FORK: requires in->pos % 64 == 0 and out != in (no overlap).  Absorbs all T rows,
 *   writes o rows [0, T) and leaves `in` unchanged; out->pos = in->pos + T.
 *
 * In both modes the arithmetic boundaries are the absolute multiples of 64 only, so a
 * replay split into several calls gives the same bits as one call.
 * x [T][C], g/beta [T][Hv], o [T][Hv][d_v] device; rows_done may be NULL.  ws must hold
 * gdn_workspace_bytes(desc, T, 1) bytes (device).  Both states' tags must match.  o, the
 * workspace bytes used and the out state may overlap none of the other buffers of the call
 * (GDN_EALIAS), apart from out being in itself in a commit. */
gdn_status gdn_prefill_chunked(const gdn_desc *desc, const void *x, const void *conv_w,
                               const float *g, const float *beta, const gdn_state *in,
                               gdn_state *out, void *o, int64_t T, int32_t mode,
                               int64_t *rows_done, void *ws, size_t ws_bytes, void *stream);

/* gdn_prefill_chunked plus per-kernel timing, for benchmarks.  events[0 .. n_events) are
 * hipEvent_t handles the caller created with timing enabled; the library records
 * events[2k] before and events[2k+1] after the k-th kernel it enqueues on `stream`
 * (k = 0 the prep kernel, 1 the chain kernel, which also writes the new conv window; pair 2
 * is recorded back to back and brackets no kernel; pairs past n_events / 2 are not
 * recorded).  Results and errors are those of gdn_prefill_chunked. */
gdn_status gdn_prefill_chunked_events(const gdn_desc *desc, const void *x, const void *conv_w,
                                      const float *g, const float *beta, const gdn_state *in,
                                      gdn_state *out, void *o, int64_t T, int32_t mode,
                                      int64_t *rows_done, void *ws, size_t ws_bytes,
                                      void *stream, void *const *events, int32_t n_events);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gdn_prefill_chunked with the workspace in a static
 * device array of GDN_NOALLOC_WORKSPACE_BYTES that the library holds on every GPU it runs on
 * until the process ends (32 MiB: about 2,200 rows of a 16/32/128 layer, enough for a pending
 * tail plus a question).  Arguments, results and refusals are gdn_prefill_chunked's; a call
 * whose rows need more workspace than the array (gdn_workspace_bytes(desc, rows, 1) >
 * GDN_NOALLOC_WORKSPACE_BYTES) is refused with GDN_EWORKSPACE and enqueues nothing.  The
 * library allocates nothing here; `stream` must belong to the current device.  Every call on
 * one GPU uses the same array: calls that overlap in time on one GPU (other streams or
 * threads) race, so a caller serialises them.  GDN_EDEVICE if the array's address cannot be
 * had. */
#define GDN_NOALLOC_WORKSPACE_BYTES (32u << 20)
gdn_status gdn_prefill_chunked_noalloc(const gdn_desc *desc, const void *x, const void *conv_w,
                                       const float *g, const float *beta, const gdn_state *in,
                                       gdn_state *out, void *o, int64_t T, int32_t mode,
                                       int64_t *rows_done, void *stream);

/* Batched branch continuation (PR "qwen3_5: run prompts that share prefixes once per prefix",
 * section Purpose: each prefix runs once up to its last multiple of 64 rows, and every branch
 * continues from the shared fp32 state and conv window with the remainder at its head; section
 * "Test Plan": branches equal plain passes over their full prompts): B sequences packed along
 * rows.  Branch b owns rows
 * [cu_rows[b], cu_rows[b+1]) of x, g, beta and o (cu_rows is a host array of B+1
 * non-decreasing offsets starting at 0; every branch has >= 1 row) and starts from
 * init[b], whose pos must be a multiple of 64.  init entries may repeat (a shared prefix
 * state, read only).  out may be NULL (no final states), else out[b] receives branch b's
 * final state; no out[b] may overlap any init state or another out, and o, the workspace
 * bytes used and the out states may overlap none of x, g, beta, conv_w or each other
 * (GDN_EALIAS).  ws must hold gdn_workspace_bytes(desc, cu_rows[B], B) bytes.  Each branch's rows and final state
 * are bitwise those of a single-sequence gdn_prefill_chunked(GDN_FORK) from init[b]. */
gdn_status gdn_prefill_branches(const gdn_desc *desc, int32_t B, const int64_t *cu_rows,
                                const void *x, const void *conv_w, const float *g,
                                const float *beta, const gdn_state *const *init,
                                gdn_state *const *out, void *o, void *ws, size_t ws_bytes,
                                void *stream);

/* ---------------------------------------------------------------- decode */

/* One-token step of B sequences, each from its own state: the width-W conv with the window
 * carried, the L2 norm of q and k, then for every value head one step of the gated delta
 * rule in fp32,
 *   S <- e^g (I - beta k k^T) S + beta k v^T,   o = scale S^T q,
 * the per-token rule the chunked prefill reaches by its chunk algebra.  It is the step that
 * follows a fork's prefill when the small model answers on top of a session ("The shadow
 * reader", section "Who asks": the fork decodes token by token, eagerly).
 *
 * x [B][C] (one row per sequence), g/beta [B][Hv], o [B][Hv][d_v] device; S must be
 * 16-byte aligned here (the step moves it in 16-byte pieces).  in[b] is read,
 * out[b] receives the advanced state (pos = in[b]->pos + 1, the tag kept); out[b] may be
 * in[b] itself (in place).  in entries may repeat (a shared read-only state), but no out[b]
 * may overlap an in[j] or out[j] of another sequence, o may overlap no input or state, and
 * no out[b] may overlap x, g, beta or conv_w (GDN_EALIAS).  There is no position
 * constraint: a decoded state sits off the 64-row grid, so only further decode steps
 * continue it (a prefill refuses it with GDN_EGRID).  The result matches the per-token rule
 * to fp32 rounding; it is not bitwise a GDN_FORK prefill of the same row, whose chunk
 * algebra rounds differently.  One kernel per group of at most 32 sequences, plus a
 * window-shift kernel when some out[b] shares its window with in[b] (in place): ping-pong
 * between two states per session to keep one launch per step.  The call enqueues kernels
 * only (no copy, fill or synchronisation), so a serving loop can capture a run of steps in a
 * HIP graph and replay it; the host-side pos fields then advance only with eager calls. */
gdn_status gdn_decode_step(const gdn_desc *desc, int32_t B, const void *x, const void *conv_w,
                           const float *g, const float *beta, const gdn_state *const *in,
                           gdn_state *const *out, void *o, void *stream);

/* ---------------------------------------------------------------- projections */

/* y[T][N] = x[T][K] w[N][K]^T: the projections around the layer (hidden -> q|k|v|gate logits,
 * and the output side), bf16 x and w, fp32 accumulation, y in out_dtype (GDN_BF16 or
 * GDN_F32).  One tiling and one summation order over K for every T, so each row of y depends
 * only on its row of x and on w: a run over any subset or grouping of rows gives the same
 * bits as a run over all of them (PR "qwen3_5: run prompts that share prefixes once per
 * prefix", section Purpose, "GEMMs": one fixed algorithm per weight shape, so grouped runs
 * equal a plain pass bit for bit).  Requires K % 64 == 0, N % 16 == 0, T >= 0 (T == 0 does
 * nothing); x, w, y device pointers, 16-byte aligned; y may overlap neither x nor w
 * (GDN_EALIAS).  Asynchronous on `stream`. */
gdn_status gdn_linear(int64_t T, int32_t K, int32_t N, const void *x, const void *w, void *y,
                      int32_t out_dtype, void *stream);

/* ---------------------------------------------------------------- full-attention layers */

/* The hybrid's full-attention layers: causal softmax attention of a call's query rows over the
 * key/value cache, with grouped key heads. */
typedef struct {
    int32_t n_q_heads, n_kv_heads; /* n_q_heads % n_kv_heads == 0; the ratio is 1, 2, 4 or a
                                      multiple of 8 */
    int32_t head_dim;              /* 128 or 256 */
    int32_t out_dtype;             /* GDN_BF16 or GDN_F32 */
    float scale;                   /* score scale (finite, > 0), usually head_dim^-1/2 */
} gdn_attn_desc;

typedef struct {
    const void *q; /* [T][n_q_heads][head_dim] bf16: the call's query rows */
    const void *k; /* [pos0 + T][n_kv_heads][head_dim] bf16: the key cache, the call's own
                      rows already appended; rows past pos0 + T are never read */
    const void *v; /* the value cache, laid out like k */
    void *o;       /* [T][n_q_heads][head_dim] out_dtype; must not overlap q, k or v */
    int64_t pos0;  /* absolute position of q's first row (rows 0 .. pos0 - 1 are cached) */
    int64_t T;     /* query rows of the call (0: nothing to do) */
} gdn_attn_seq;

/* o = softmax(scale q K^T, keys 0 .. p for the query at absolute position p) V for every row of
 * every sequence, query head h reading key head h / (n_q_heads / n_kv_heads).  Split-K flash
 * attention as the pages run it ("Long context and sessions", section "The KV cache"): key
 * positions in splits of 256 at absolute multiples of 256, an online softmax that folds the
 * splits into a running max, sum and accumulator in ascending order, so each output row depends
 * only on its absolute position and the cache contents: cutting a prompt into calls at any row,
 * or running branches over a shared cached prefix, gives the same bits as one call over the
 * whole prompt.  Rewinding needs no checkpoint: a later call from any pos0 reuses cache rows
 * below pos0 as they are ("The shadow reader", section "Exact on a grid").  fp32 scores,
 * softmax and accumulation; the softmax weights meet V as bf16.  All pointers device, 16-byte
 * aligned.  B >= 0 sequences (an array on the host), cut into launches of at most 32.
 * Asynchronous on `stream`.  GDN_EINVAL / GDN_ESHAPE / GDN_EALIAS on bad arguments, nothing
 * enqueued. */
gdn_status gdn_attention_prefill(const gdn_attn_desc *desc, int32_t B, const gdn_attn_seq *seqs,
                                 void *stream);

/* ---------------------------------------------------------------- host scheduling (no device) */

/* Rows a COMMIT from an aligned position absorbs out of n available rows:
 * floor(n / grid) * grid ("The shadow reader", section "Exact on a grid"). -1 on bad args. */
int64_t gdn_commit_rows(int64_t n, int32_t grid);

/* Rows a shared prefix that ends at absolute row `prefix_end` runs from a state at
 * `state_pos` (a multiple of 64): max(0, floor(prefix_end / 64) * 64 - state_pos).  The
 * remaining prefix_end - state_pos - run rows run at the head of every later group or
 * branch (PR "qwen3_5: run prompts that share prefixes once per prefix", section Purpose,
 * "Split points").  -1 on bad args. */
int64_t gdn_shared_prefix_rows(int64_t state_pos, int64_t prefix_end);

/* Checkpoint ring: at most `cap` (<= GDN_MAX_CHECKPOINTS) checkpoints, each at a
 * committed position, held in caller-owned state slots 0..cap-1 ("The shadow reader",
 * sections "One session's state" and "Exact on a grid"). */
typedef struct {
    int32_t cap, n;
    int64_t pos[GDN_MAX_CHECKPOINTS];  /* pos[i] of slot i, -1 when empty */
    uint64_t age[GDN_MAX_CHECKPOINTS]; /* insertion stamp of slot i */
    uint64_t clock;
} gdn_ckpt_ring;

gdn_status gdn_ckpt_init(gdn_ckpt_ring *ring, int32_t cap);
/* Slot to capture a checkpoint at `pos` into: the slot already holding pos, else an empty
 * slot, else the oldest one (evicted).  Records pos.  -1 on bad args. */
int32_t gdn_ckpt_push(gdn_ckpt_ring *ring, int64_t pos);
/* Slot of the newest checkpoint with pos <= d (the largest such pos), or -1 if none:
 * then start over from a zero state. */
int32_t gdn_ckpt_find(const gdn_ckpt_ring *ring, int64_t d);
/* Forget every checkpoint with pos > d (they no longer describe the prompt).  Returns the
 * number dropped. */
int32_t gdn_ckpt_drop_above(gdn_ckpt_ring *ring, int64_t d);

/* Static text of a status code. */
const char *gdn_status_str(gdn_status status);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
