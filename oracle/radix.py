"""Hybrid prefix cache: what a lookup must return (brute force).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source passages
---------------
* 24-ai.news TokenSpeed article, optimisation list, hybrid prefix caching
  for GDN/Mamba: the logical cache lives in C++, the tensors elsewhere;
  cached prefixes are found by radix-tree matching with Mamba-slot
  attachments, and cached states are reused with copy-on-write semantics.
* zubnet.ai TokenSpeed article, second paragraph: the recurrent state is
  checkpointed next to the KV; cached checkpoints are reused without
  mutation.

Reading (the pages name the mechanism, not its rules): a request of a
hybrid model can resume only at a prefix for which both the KV and the
recurrent state were saved, so a lookup returns the longest saved prefix
(a sequence that was inserted with a state) that begins the query, with
that state's slot; length 0 (the zero state) when none.  When the same
token sequence is saved twice, the first saved state stays.  This model is
the definition written as a scan over every saved sequence; it knows
nothing of trees, nodes or pages.  Which physical pages back a match is
not unique (a shared page may come from any sequence that wrote the same
tokens), so tests check the pages by content instead.
"""


class PrefixCacheModel:
    def __init__(self):
        self.saved = {}  # token tuple -> slot of the first save with a state

    def insert(self, tokens, slot):
        key = tuple(int(t) for t in tokens)
        if slot >= 0 and len(key) > 0 and key not in self.saved:
            self.saved[key] = int(slot)

    def match(self, tokens):
        """(length, slot) of the longest saved sequence that begins `tokens`."""
        q = tuple(int(t) for t in tokens)
        best, slot = 0, -1
        for key, s in self.saved.items():
            if len(key) > best and q[:len(key)] == key:
                best, slot = len(key), s
        return best, slot
