"""CPU oracle for the paged-cache updates around a verify step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module; the product path never calls it.
It shares no code with the HIP library and imports nothing from it.

What it follows:

* "Kimi K3: DSpark speculative decoding under Helix CP", first commit message
  ("Per-token primitive", "mla_rope_generation") and the same items under
  "Changes": every token of a verify group (1 target + k drafts) has its own
  rank-local KV write slot, -1 when another rank owns the position, and this
  per-token slot table decides which tokens the KV append writes.
* "Kimi K3 support with DSpark speculative decoding", "What does this PR do?",
  "Speculative decoding": after verification the KV cache trims the rejected
  tail of the group.

Readings where the pages are silent (each is listed in the design notes):

* a slot is a request-logical key position j, the same index the attention
  uses: key j of request b lives at page block_table[b, j // 64], row j % 64;
* the latent is written unchanged (NoPE: there is no rotary part to apply);
* a slot below -1 or at least P*64, or a page id outside [0, N), is an error:
  nothing is written and the token is counted;
* the trim keeps the target token and the accepted drafts, the kept tokens
  being the first of the group (verification accepts a prefix of the
  drafts), so the request loses its last T - 1 - accepted keys;
* a page that holds only dropped keys is released: its block-table entry
  becomes -1 and its id is reported (-1 when no page is released).

Everything is plain Python loops over the tokens and requests, on integer
page/slot arithmetic and exact bf16 bit patterns: there is no floating point
here at all.
"""
from __future__ import annotations

import numpy as np

PAGE = 64


def kv_append(pool_bits, block_table, slots, new_latent_bits):
    """The pool after the append, and the number of rejected tokens.

    pool_bits [N, 64, 512] uint16, block_table [B, P] int32, slots [B, T]
    int32, new_latent_bits [B, T, 512] uint16.  Tokens are applied in (b, t)
    order, so with a duplicated slot the last one wins here (the library
    leaves that order unspecified; tests use distinct slots or accept either).
    """
    pool = np.array(pool_bits, dtype=np.uint16, copy=True)
    block_table = np.asarray(block_table)
    slots = np.asarray(slots)
    n_pages = pool.shape[0]
    n_batch, n_tok = slots.shape
    max_keys = block_table.shape[1] * PAGE
    bad = 0
    for b in range(n_batch):
        for t in range(n_tok):
            slot = int(slots[b, t])
            if slot == -1:
                continue   # owned by another rank: nothing to write here
            if slot < 0 or slot >= max_keys:
                bad += 1
                continue
            page = int(block_table[b, slot // PAGE])
            if page < 0 or page >= n_pages:
                bad += 1
                continue
            pool[page, slot % PAGE, :] = new_latent_bits[b, t, :]
    return pool, bad


def kv_trim(kv_len, accepted, block_table, q_len):
    """(new_len [B], block_table after the trim [B, P], released_page [B]).

    Request b held kv_len[b] keys with its group of q_len tokens last; it keeps
    the target and a = clamp(accepted[b], 0, q_len - 1) drafts.
    """
    table = np.array(block_table, dtype=np.int32, copy=True)
    n_batch, max_pages = table.shape
    new_len = np.zeros(n_batch, dtype=np.int32)
    released = np.full(n_batch, -1, dtype=np.int32)
    for b in range(n_batch):
        length = min(max(int(kv_len[b]), 0), max_pages * PAGE)
        kept_drafts = min(max(int(accepted[b]), 0), q_len - 1)
        dropped = q_len - 1 - kept_drafts
        new = max(0, length - dropped)
        new_len[b] = new
        # pages all of whose keys were dropped: first key 64 p in [new, length)
        emptied = [p for p in range(max_pages) if new <= PAGE * p < length]
        assert len(emptied) <= 1, "fewer than 64 keys are dropped, so at most one page empties"
        for p in emptied:
            released[b] = table[b, p]
            table[b, p] = -1
    return new_len, table, released
