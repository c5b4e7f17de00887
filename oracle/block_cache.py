"""Oracle: the device-side block cache's residency policy, as a plain sequential model.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this module.  It shares no code with the HIP library.

Follows Strata compare v0.1.2...v0.1.6, "KV streaming for the QSA layers" (``kv_stream.hpp``
header comment and ``kv_stream.cu``): the authoritative K/V sit in pinned host memory; device
memory holds ``n_slots`` pages of ``page_size`` cells; ``page_table[page]`` is the slot holding
the page, or -1.  Before a read, every page a selection names is made resident:

1. a page already resident gets this call's epoch and its reference bit; a missing page is
   claimed once (a page named several times is one miss);
2. one victim slot per miss is taken by a CLOCK sweep (second chance) starting at the hand:
   a slot this call uses is never taken; a free slot or one whose reference bit is clear is
   taken; any other slot the hand passes loses its reference bit; the hand stops just past
   the last slot taken, and gives up after three turns (overflow);
3. the table is re-pointed (the victim's old page becomes absent, the new page points at it),
   and the missed pages are copied from the host copy into their slots.

Counters: misses (pages placed), lookups (one per entry whose predecessor in the same
selection names another page), calls.  Which missed page lands in which of this call's victim
slots follows the order in which the device claims them and is not fixed by the policy;
``resolve`` therefore returns the victim set, and ``adopt`` takes the device's actual pairing
so that later calls are modelled exactly.
"""
from __future__ import annotations


class ClockCache:
    def __init__(self, n_pages: int, n_slots: int, page_size: int):
        self.n_pages, self.n_slots, self.page_size = n_pages, n_slots, page_size
        self.reset()

    def reset(self):
        self.page_table = [-1] * self.n_pages
        self.slot_page = [-1] * self.n_slots
        self.slot_stamp = [-1] * self.n_slots
        self.slot_ref = [0] * self.n_slots
        self.epoch = 0
        self.hand = 0
        self.misses = self.lookups = self.calls = 0
        self.overflow = False

    def pages_of(self, selections):
        """Distinct pages in first-named order, and the lookup count: an entry counts unless the
        entry just before it in the same selection names the same page (padding -1 never counts
        and ends a run)."""
        seen, order, lookups = set(), [], 0
        for sel in selections:
            prev = None
            for c in sel:
                c = int(c)
                if c < 0:
                    prev = None
                    continue
                p = c // self.page_size
                if p != prev:
                    lookups += 1
                prev = p
                if p not in seen:
                    seen.add(p)
                    order.append(p)
        return order, lookups

    def resolve(self, selections):
        """One call.  Returns (victim slots in hand order, pages missed this call, overflow)."""
        self.epoch += 1
        pages, lookups = self.pages_of(selections)
        missed = []
        for p in pages:
            s = self.page_table[p]
            if s >= 0:
                self.slot_stamp[s] = self.epoch
                self.slot_ref[s] = 1
            else:
                missed.append(p)
        need = min(len(missed), self.n_slots)
        victims = []
        j, passed = self.hand, 0
        while len(victims) < need and passed < 3 * self.n_slots:
            mine = self.slot_stamp[j] == self.epoch
            if not mine and (self.slot_page[j] < 0 or self.slot_ref[j] == 0):
                victims.append(j)
                self.slot_stamp[j] = self.epoch
            elif not mine:
                self.slot_ref[j] = 0
            j = (j + 1) % self.n_slots
            passed += 1
        if victims:
            self.hand = (victims[-1] + 1) % self.n_slots
        else:
            self.hand = j
        placed = len(victims)
        overflow = placed < len(missed)
        # default pairing (claim order == hand order); the device may pair differently
        for p, s in zip(missed, victims):
            old = self.slot_page[s]
            if old >= 0:
                self.page_table[old] = -1
            self.slot_page[s] = p
            self.slot_stamp[s] = self.epoch
            self.slot_ref[s] = 1
            self.page_table[p] = s
        self.misses += placed
        self.lookups += lookups
        self.calls += 1
        self.overflow = self.overflow or overflow
        return victims, missed[:placed], overflow

    def adopt(self, page_table, slot_page):
        """Take the device's page -> slot pairing of the pages placed so far."""
        self.page_table = [int(x) for x in page_table]
        self.slot_page = [int(x) for x in slot_page]

    def rows(self, selection):
        """Slot-pool rows of a selection of cells (-1 stays -1; an absent page gives -1)."""
        out = []
        for c in selection:
            c = int(c)
            if c < 0:
                out.append(-1)
                continue
            s = self.page_table[c // self.page_size]
            out.append(-1 if s < 0 else s * self.page_size + c % self.page_size)
        return out
