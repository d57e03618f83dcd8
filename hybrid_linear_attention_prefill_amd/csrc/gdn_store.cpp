// gdn_store.cpp -- session store: resident states under a byte cap, least recently used sessions
// spilled to files and read back exactly ("The shadow reader", section "Memory and the disk":
// resident states are capped; past the cap the least recently used session goes to disk and
// comes back exact when it is fed again, and without a disk it is dropped and read again from
// the start; a planned stop writes every resident session; "Long context and sessions", section
// "Sessions on one engine": a session is brought back from a GPU slot, from disk, or fresh).
//
// Host code only (no ROCm header): the device is reached through gdn_state_save / gdn_state_load
// and gdn_state_init.  All memory is the caller's: the device slots and the entry table.
#include <cerrno>
#include <cstdio>
#include <cstring>

#include "gdn_internal.h"

namespace {

bool store_ok(const gdn_store *s)
{
    return s && s->slots && s->entries && s->n_slots > 0 && s->max_entries > 0 &&
           s->max_resident > 0 && s->max_resident <= s->n_slots && gdn_desc_check(&s->desc) == GDN_OK;
}

// File of session `id`: <dir>/gdn-<id as 16 hex digits>.state
bool path_of(const gdn_store *s, uint64_t id, char *out, size_t n)
{
    const int k = std::snprintf(out, n, "%s/gdn-%016llx.state", s->dir, (unsigned long long)id);
    return k > 0 && (size_t)k < n;
}

int32_t find_entry(const gdn_store *s, uint64_t id)
{
    for (int32_t i = 0; i < s->max_entries; ++i)
        if (s->entries[i].where != GDN_STORE_UNUSED && s->entries[i].id == id) return i;
    return -1;
}

int32_t n_resident(const gdn_store *s)
{
    int32_t n = 0;
    for (int32_t i = 0; i < s->max_entries; ++i) n += s->entries[i].where == GDN_STORE_RESIDENT;
    return n;
}

// Moves resident entry e out of its slot: to its file when the store has a directory and the
// write succeeds (ON_DISK), else DROPPED (its file, if any, removed: a failed write leaves no
// stale file).  The slot's state holds the session's latest pos.
gdn_status spill(gdn_store *s, int32_t e, void *stream)
{
    gdn_store_entry &en = s->entries[e];
    gdn_state &slot = s->slots[en.slot];
    en.pos = slot.pos;
    char path[sizeof(s->dir) + 40];
    bool written = false;
    if (s->dir[0] && path_of(s, en.id, path, sizeof(path))) {
        const gdn_status st = gdn_state_save(&s->desc, &slot, s->weights_hash, path, stream);
        if (st == GDN_EDEVICE) return st;  // the slot stays resident
        written = st == GDN_OK;
        if (!written) std::remove(path);
    }
    en.where = written ? GDN_STORE_ON_DISK : GDN_STORE_DROPPED;
    if (!written) en.pos = 0;
    en.slot = -1;
    return GDN_OK;
}

int32_t lru_resident(const gdn_store *s)
{
    int32_t best = -1;
    for (int32_t i = 0; i < s->max_entries; ++i)
        if (s->entries[i].where == GDN_STORE_RESIDENT &&
            (best < 0 || s->entries[i].last_use < s->entries[best].last_use))
            best = i;
    return best;
}

}  // namespace

extern "C" {

gdn_status gdn_store_init(gdn_store *s, const gdn_desc *desc, gdn_state *slots, int32_t n_slots,
                          size_t cap_bytes, const char *dir, uint64_t weights_hash,
                          gdn_store_entry *entries, int32_t max_entries)
{
    if (!s || !desc || !slots || !entries || n_slots <= 0 || max_entries < n_slots)
        return GDN_EINVAL;
    gdn_status st = gdn_desc_check(desc);
    if (st) return st;
    const size_t one = gdn_state_S_bytes(desc) + gdn_state_conv_bytes(desc);
    const size_t fit = cap_bytes / one;
    if (fit == 0) return GDN_EINVAL;
    if (dir && std::strlen(dir) >= sizeof(s->dir)) return GDN_EINVAL;
    for (int32_t i = 0; i < n_slots; ++i)
        if (!slots[i].S || (desc->conv_width > 0 && !slots[i].conv)) return GDN_EINVAL;
    std::memset(s, 0, sizeof(*s));
    s->desc = *desc;
    s->slots = slots;
    s->n_slots = n_slots;
    s->cap_bytes = cap_bytes;
    s->state_bytes = one;
    s->max_resident = (int32_t)(fit < (size_t)n_slots ? fit : (size_t)n_slots);
    s->entries = entries;
    s->max_entries = max_entries;
    s->weights_hash = weights_hash;
    if (dir) std::strcpy(s->dir, dir);
    for (int32_t i = 0; i < max_entries; ++i) {
        std::memset(&entries[i], 0, sizeof(entries[i]));
        entries[i].where = GDN_STORE_UNUSED;
        entries[i].slot = -1;
    }
    return GDN_OK;
}

gdn_status gdn_store_acquire(gdn_store *s, uint64_t id, gdn_state **state, int32_t *origin,
                             void *stream)
{
    if (!store_ok(s) || !state || !origin) return GDN_EINVAL;
    int32_t e = find_entry(s, id);
    if (e >= 0 && s->entries[e].where == GDN_STORE_RESIDENT) {
        s->entries[e].last_use = ++s->clock;
        *state = &s->slots[s->entries[e].slot];
        *origin = GDN_STORE_WAS_RESIDENT;
        return GDN_OK;
    }
    if (e < 0) {  // a new session: a free entry, else the least recently used one not resident
        for (int32_t i = 0; i < s->max_entries && e < 0; ++i)
            if (s->entries[i].where == GDN_STORE_UNUSED) e = i;
        if (e < 0)
            for (int32_t i = 0; i < s->max_entries; ++i)
                if (s->entries[i].where != GDN_STORE_RESIDENT &&
                    (e < 0 || s->entries[i].last_use < s->entries[e].last_use))
                    e = i;
        if (e < 0) return GDN_EINVAL;  // every entry resident: the table is smaller than the slots
        if (s->entries[e].where == GDN_STORE_ON_DISK) {
            char path[sizeof(s->dir) + 40];
            if (path_of(s, s->entries[e].id, path, sizeof(path))) std::remove(path);
        }
        gdn_store_entry &en = s->entries[e];
        en.id = id;
        en.pos = 0;
        en.where = GDN_STORE_DROPPED;  // nothing stored yet: starts fresh
        en.slot = -1;
    }
    // a slot: a free one, else the least recently used resident session's
    int32_t slot = -1;
    if (n_resident(s) < s->max_resident) {
        for (int32_t k = 0; k < s->n_slots && slot < 0; ++k) {
            bool taken = false;
            for (int32_t i = 0; i < s->max_entries && !taken; ++i)
                taken = s->entries[i].where == GDN_STORE_RESIDENT && s->entries[i].slot == k;
            if (!taken) slot = k;
        }
    }
    if (slot < 0) {
        const int32_t v = lru_resident(s);
        if (v < 0) return GDN_EINVAL;
        slot = s->entries[v].slot;
        gdn_status st = spill(s, v, stream);
        if (st) return st;
    }
    gdn_store_entry &en = s->entries[e];
    gdn_state *dst = &s->slots[slot];
    int32_t from = GDN_STORE_FRESH;
    if (en.where == GDN_STORE_ON_DISK) {
        char path[sizeof(s->dir) + 40];
        if (path_of(s, id, path, sizeof(path))) {
            const gdn_status st = gdn_state_load(&s->desc, dst, s->weights_hash, path, stream);
            if (st == GDN_EDEVICE) return st;
            if (st == GDN_OK) from = GDN_STORE_FROM_DISK;
            else std::remove(path);  // unreadable, damaged or for other weights / grid: read again
        }
    }
    if (from == GDN_STORE_FRESH) {
        gdn_status st = gdn_state_init(&s->desc, dst, stream);
        if (st) return st;
    }
    en.where = GDN_STORE_RESIDENT;
    en.slot = slot;
    en.pos = dst->pos;
    en.last_use = ++s->clock;
    *state = dst;
    *origin = from;
    return GDN_OK;
}

gdn_status gdn_store_evict(gdn_store *s, uint64_t id, void *stream)
{
    if (!store_ok(s)) return GDN_EINVAL;
    const int32_t e = find_entry(s, id);
    if (e < 0) return GDN_EINVAL;
    if (s->entries[e].where != GDN_STORE_RESIDENT) return GDN_OK;
    return spill(s, e, stream);
}

gdn_status gdn_store_flush(gdn_store *s, void *stream)
{
    if (!store_ok(s)) return GDN_EINVAL;
    if (!s->dir[0]) return GDN_OK;
    for (int32_t i = 0; i < s->max_entries; ++i) {
        gdn_store_entry &en = s->entries[i];
        if (en.where != GDN_STORE_RESIDENT) continue;
        char path[sizeof(s->dir) + 40];
        if (!path_of(s, en.id, path, sizeof(path))) return GDN_EFILE;
        en.pos = s->slots[en.slot].pos;
        const gdn_status st = gdn_state_save(&s->desc, &s->slots[en.slot], s->weights_hash, path, stream);
        if (st) return st;
    }
    return GDN_OK;
}

gdn_status gdn_store_drop(gdn_store *s, uint64_t id)
{
    if (!store_ok(s)) return GDN_EINVAL;
    const int32_t e = find_entry(s, id);
    if (e < 0) return GDN_OK;
    char path[sizeof(s->dir) + 40];
    if (s->dir[0] && path_of(s, id, path, sizeof(path))) std::remove(path);
    std::memset(&s->entries[e], 0, sizeof(s->entries[e]));
    s->entries[e].where = GDN_STORE_UNUSED;
    s->entries[e].slot = -1;
    return GDN_OK;
}

int32_t gdn_store_find(const gdn_store *s, uint64_t id)
{
    if (!store_ok(s)) return -1;
    return find_entry(s, id);
}

}  // extern "C"
