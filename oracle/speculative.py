"""Draft-verify bookkeeping: rollback by index, no copies.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source passages
---------------
* zubnet.ai TokenSpeed article, second paragraph: during speculative
  decoding the engine redirects an index array (``current_input_indices``)
  instead of copying tensors, and cached checkpoints are reused without
  mutation (copy-on-write).
* 24-ai.news TokenSpeed article, optimisation list, "Mamba State Update":
  the state update becomes an O(1) pointer update.

Reading (pages silent on the protocol): a verify step appends T draft tokens
(KV reserved for L0 .. L0+T-1, GDN state after each draft checkpointed into
its own freshly acquired slot out_slots[t]); the host then keeps the first
``accepted`` drafts, 0 <= accepted <= T, with no bonus token:

* KV: the sequence is truncated to L0 + accepted (pages past the end go back
  to the free list; stale K/V left inside a kept partial page is masked by
  the sequence length).
* State: the current slot becomes in_slot when accepted == 0, otherwise
  out_slots[accepted - 1].  Every other out slot is released, in draft order;
  then, if accepted > 0 and in_slot >= 0, the sequence's reference to
  in_slot is released (in_slot = -1 stands for the zero state, no slot).
* Every precondition is checked before anything changes (a failed call
  leaves both models untouched).
"""


def rollback(pt, slots, sid, T, accepted, in_slot, out_slots):
    """Apply the accept decision to a PageTableModel and a SlotPoolModel.

    Returns the slot holding the sequence's current state.
    """
    from .paging import ModelError

    if not (0 <= accepted <= T) or len(out_slots) != T:
        raise ModelError("invalid")
    L = pt.seqs[sid]["len"] if sid in pt.seqs else None
    if L is None:
        raise ModelError("bad_seq")
    if L < T:
        raise ModelError("range")
    if len(set(out_slots)) != T:
        raise ModelError("invalid")
    for x in out_slots:
        if not (0 <= x < slots.n) or slots.ref[x] == 0 or x == in_slot:
            raise ModelError("bad_slot")
    if accepted > 0 and in_slot >= 0 and (in_slot >= slots.n or slots.ref[in_slot] == 0):
        raise ModelError("bad_slot")
    pt.truncate(sid, L - T + accepted)
    keep = in_slot if accepted == 0 else out_slots[accepted - 1]
    for t in range(T):
        if t != accepted - 1:
            slots.release(out_slots[t])
    if accepted > 0 and in_slot >= 0:
        slots.release(in_slot)
    return keep
