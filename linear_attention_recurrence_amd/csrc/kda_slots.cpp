// kda_slots.cpp -- host side of the prefix-cache state protocol: checkpoint-aligned chunking and the
// ownership of the state pool's slots under the three state moves (copy-on-write restore, snapshot,
// donate).
//
// Sources: "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS blog), section "Hybrid KDA Memory
// Management", subsection on the three state moves: a request's live state is one working slot
// overwritten by every forward; restores and snapshots are copies on the one forward stream; snapshots
// go to a ping-pong pair whose second slot exists only around a snapshot; caching donates the latest
// snapshot's slot index to the radix tree (no bytes move) and a fresh slot backfills, so a snapshot
// never writes the slot a donate handed out. Kimi K3 B200 deployment notes (zdszero.github.io), the
// CuTe FlashKDA prefill item: the prefix cache checkpoints the state every 256 tokens, so chunks other
// than a request's last are cut to multiples of 256 and the state at a chunk's end is a checkpoint.
//
// Every slot has exactly one owner: the free list, one open request (its working slot or its latest
// snapshot, plus the fresh target during a snapshot), or the tree. The functions below change owners
// and return the copies to enqueue (kda_state_move); they never touch device memory.
#include <cstdint>
#include <new>
#include <vector>

#include "../../include/kda.h"
#include "kda_internal.h"

struct kda_slots {
  std::vector<int32_t> owner;  // kFree, kTree or the id (>= 0) of the request that holds the slot
  std::vector<int32_t> free_list;
  int32_t next_id = 0;
  static constexpr int32_t kFree = -1, kTree = -2;

  int32_t take(int32_t id) {
    const int32_t s = free_list.back();
    free_list.pop_back();
    owner[s] = id;
    return s;
  }
  void give_back(int32_t s) {
    owner[s] = kFree;
    free_list.push_back(s);
  }
  bool valid(int32_t s) const { return s >= 0 && s < (int32_t)owner.size(); }
  // the request's slots, as this pool recorded them
  bool holds(const kda_request_slots* r) const {
    return r && r->id >= 0 && valid(r->working) && owner[r->working] == r->id &&
           (r->snap == -1 || (valid(r->snap) && owner[r->snap] == r->id && r->snap != r->working));
  }
};

extern "C" {

kda_status kda_chunk_split(int64_t pos0, int64_t len, int64_t budget, int64_t align, int64_t* lens_host,
                           int max_chunks, int* n_chunks) {
  if (!n_chunks || pos0 < 0 || len < 0 || budget < 1 || align < 1 || max_chunks < 0 || (max_chunks > 0 && !lens_host))
    return kda::fail(KDA_ERR_INVALID_ARG, "kda_chunk_split: bad pos0/len/budget/align/max_chunks");
  int n = 0;
  int64_t pos = pos0;
  const int64_t end = pos0 + len;
  while (pos < end) {
    int64_t stop;
    if (end - pos <= budget) {
      stop = end;  // the last chunk takes the rest
    } else {
      stop = (pos + budget) / align * align;  // the last checkpoint boundary within the budget
      if (stop <= pos) stop = pos + budget;   // none within it: a full budget, without a checkpoint
    }
    if (n < max_chunks) lens_host[n] = stop - pos;
    ++n;
    pos = stop;
  }
  *n_chunks = n;
  if (n > max_chunks) return kda::fail(KDA_ERR_INVALID_ARG, "kda_chunk_split: more chunks than max_chunks (count in *n_chunks)");
  return kda::ok();
}

kda_status kda_slots_create(int n_slots, kda_slots** out) {
  if (!out || n_slots < 1) return kda::fail(KDA_ERR_INVALID_ARG, "kda_slots_create: n_slots >= 1 and out are required");
  *out = nullptr;
  kda_slots* p = new (std::nothrow) kda_slots();
  if (!p) return kda::fail(KDA_ERR_HOST_ALLOC, "kda_slots_create: out of host memory");
  try {
    p->owner.assign(n_slots, kda_slots::kFree);
    p->free_list.reserve(n_slots);
    for (int s = n_slots - 1; s >= 0; --s) p->free_list.push_back(s);  // slot 0 handed out first
  } catch (...) {
    delete p;
    return kda::fail(KDA_ERR_HOST_ALLOC, "kda_slots_create: out of host memory");
  }
  *out = p;
  return kda::ok();
}

void kda_slots_destroy(kda_slots* p) { delete p; }

int kda_slots_free_count(const kda_slots* p) { return p ? (int)p->free_list.size() : -1; }

int kda_slots_owner(const kda_slots* p, int32_t slot) {
  if (!p || !p->valid(slot)) return -3;
  return p->owner[slot];
}

kda_status kda_request_open(kda_slots* p, int32_t cached_slot, kda_request_slots* r, kda_move* restore_host,
                            int* n_moves) {
  if (!p || !r || !n_moves) return kda::fail(KDA_ERR_INVALID_ARG, "kda_request_open: pool, r and n_moves are required");
  if (cached_slot != -1 && !(p->valid(cached_slot) && p->owner[cached_slot] == kda_slots::kTree))
    return kda::fail(KDA_ERR_INVALID_ARG, "kda_request_open: a restore reads only a slot the tree owns");
  if (cached_slot != -1 && !restore_host) return kda::fail(KDA_ERR_INVALID_ARG, "kda_request_open: restore_host is required");
  if (p->free_list.empty()) return kda::fail(KDA_ERR_NO_SLOT, "kda_request_open: no free slot");
  r->id = p->next_id++;
  r->working = p->take(r->id);
  r->snap = -1;
  *n_moves = 0;
  if (cached_slot != -1) {  // copy-on-write: the tree's checkpoint stays as it is, the copy is the request's
    restore_host[0].src = cached_slot;
    restore_host[0].dst = r->working;
    *n_moves = 1;
  }
  return kda::ok();
}

kda_status kda_request_snapshot(kda_slots* p, kda_request_slots* r, kda_move* move_host) {
  if (!p || !move_host || !p->holds(r)) return kda::fail(KDA_ERR_INVALID_ARG, "kda_request_snapshot: not an open request of this pool");
  if (p->free_list.empty()) return kda::fail(KDA_ERR_NO_SLOT, "kda_request_snapshot: no free slot");
  const int32_t target = p->take(r->id);  // the pair's second slot, fresh: never the tree's or the latest
  move_host->src = r->working;
  move_host->dst = target;
  if (r->snap != -1) p->give_back(r->snap);  // superseded; later writes to it are ordered after this copy
  r->snap = target;
  return kda::ok();
}

kda_status kda_request_donate(kda_slots* p, kda_request_slots* r, int32_t* slot) {
  if (!p || !slot || !p->holds(r)) return kda::fail(KDA_ERR_INVALID_ARG, "kda_request_donate: not an open request of this pool");
  if (r->snap == -1) return kda::fail(KDA_ERR_INVALID_ARG, "kda_request_donate: no snapshot to donate");
  p->owner[r->snap] = kda_slots::kTree;  // ownership moves, no bytes; the next snapshot takes a fresh slot
  *slot = r->snap;
  r->snap = -1;
  return kda::ok();
}

kda_status kda_request_close(kda_slots* p, kda_request_slots* r) {
  if (!p || !p->holds(r)) return kda::fail(KDA_ERR_INVALID_ARG, "kda_request_close: not an open request of this pool");
  if (r->snap != -1) p->give_back(r->snap);
  p->give_back(r->working);
  r->id = -1;
  r->working = -1;
  r->snap = -1;
  return kda::ok();
}

kda_status kda_slot_release(kda_slots* p, int32_t slot) {
  if (!p || !p->valid(slot) || p->owner[slot] != kda_slots::kTree)
    return kda::fail(KDA_ERR_INVALID_ARG, "kda_slot_release: only a slot the tree owns can be released");
  p->give_back(slot);
  return kda::ok();
}

}  // extern "C"
