"""Exact integer model of a ReplaySSM sequence's buffer indices.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The explainer ("ReplaySSM for hybrid SSM-Transformer stacks",
frontier.agentik-os.com) describes per sequence a checkpoint at an earlier
token position and a ring buffer of the inputs since then ("Maintain two pieces
of SSM state"); appending moves the buffer tail, a commit folds the whole buffer
into the checkpoint and resets it ("Periodically commit a new checkpoint"), and
rejecting k speculative tokens moves the tail back by k while the checkpoint
never changes ("Cheap speculative decoding rollback").

Per sequence the model keeps

* ``pos`` -- absolute token position of the checkpoint (int64),
* ``len`` -- number of buffered entries since the checkpoint (int32).

Entry j (0-based since the checkpoint) lives in ring slot ``(pos + j) % cap``.
Invariant: ``0 <= len <= cap`` and ``pos + len`` = tokens appended - tokens
rolled back.  Reading taken where the pages are silent: rolling back further
than the checkpoint is an error, because the checkpoint cannot move backwards;
an append that would exceed the ring's capacity is an error.  Both leave the
sequence unchanged and set a sticky status bit.
"""
import numpy as np

STATUS_OVERFLOW = 1   # append / verify would exceed the ring capacity
STATUS_ROLLBACK = 2   # n_reject < 0 or n_reject > len
STATUS_NONFINITE = 4  # non-finite state met while quantising


class IndexModel:
    def __init__(self, batch: int, cap: int):
        self.cap = int(cap)
        self.pos = np.zeros(batch, dtype=np.int64)
        self.len = np.zeros(batch, dtype=np.int32)
        self.status = 0

    @property
    def batch(self) -> int:
        return self.pos.shape[0]

    def slot(self, b: int, j: int) -> int:
        """Ring slot of entry j of sequence b."""
        return int((self.pos[b] + j) % self.cap)

    def append(self, n: int = 1):
        """Append n entries to every sequence.  Returns the boolean mask of
        sequences that accepted them (the rest overflowed and are unchanged)."""
        ok = (self.len.astype(np.int64) + n) <= self.cap
        if not ok.all():
            self.status |= STATUS_OVERFLOW
        self.len[ok] += n
        return ok

    def commit(self, mask=None, min_len: int = 0):
        """Fold the whole buffer of every selected sequence with len >= min_len.
        Returns the mask of sequences whose checkpoint was rebuilt."""
        sel = self.len >= min_len
        if mask is not None:
            sel &= np.asarray(mask, dtype=bool)
        self.pos[sel] += self.len[sel]
        self.len[sel] = 0
        return sel

    def rollback(self, n_reject):
        """Move the tail of sequence b back by n_reject[b] entries."""
        n = np.asarray(n_reject, dtype=np.int64)
        ok = (n >= 0) & (n <= self.len)
        if not ok.all():
            self.status |= STATUS_ROLLBACK
        self.len[ok] -= n[ok].astype(np.int32)
        return ok

    def snapshot(self):
        return self.pos.copy(), self.len.copy()
