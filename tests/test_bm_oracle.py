"""The block-manager oracle against its pins, and planted mistakes that the pins must
catch (subclasses that break one rule each)."""
import pytest

import bm_pins as P
from oracle.blockmgr import BlockManager


@pytest.mark.parametrize("pin", P.ALL_BM_PINS, ids=lambda f: f.__name__)
def test_oracle_block_manager_pin(pin):
    pin(BlockManager)


class NoCopyOnWrite(BlockManager):
    """Writes into a shared block in place."""

    def append_token(self, sid, token_id=0):
        j = self.lengths[sid] // self.bs
        if j < len(self.tables[sid]) and self.ref[self.tables[sid][j]] > 1:
            self.ref[self.tables[sid][j]] = 1      # pretend it is private
        return super().append_token(sid, token_id)


class OwnTokensKey(BlockManager):
    """Keys a cached block by its own tokens only (the printed hash, taken literally)."""

    def add_sequence(self, sid, num_tokens, token_ids=None):
        hits = []
        if token_ids is not None:
            for j in range(num_tokens // self.bs):
                own = tuple(token_ids[j * self.bs:(j + 1) * self.bs])
                b = next((b for k, b in self.cache.items() if k[-self.bs:] == own), None)
                if b is None:
                    break
                hits.append(b)
        if not hits:
            return super().add_sequence(sid, num_tokens, token_ids)
        # share the blocks found, then place the rest as a plain prompt would
        got = super().add_sequence(sid, num_tokens, token_ids)
        for j, b in enumerate(hits):
            if self.tables[sid][j] != b:
                self._release(self.tables[sid][j])
                self._hold(b)
                self.tables[sid][j] = b
        return max(got, len(hits) * self.bs)


class EvictMostRecent(BlockManager):
    def _take(self):
        if not self.free and self.cold:
            self.cold.insert(0, self.cold.pop())
        return super()._take()


class FreeListQueue(BlockManager):
    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.cold.append(b)
            else:
                self.free.insert(0, b)          # released blocks handed out last


class ForwardRelease(BlockManager):
    def free_sequence(self, sid):
        for b in self.tables.pop(sid):
            self._release(b)
        del self.lengths[sid]
        del self.tokens[sid]


class NoTransaction(BlockManager):
    """Holds prefix hits before checking that the misses fit."""

    def add_sequence(self, sid, num_tokens, token_ids=None):
        if token_ids is not None:
            for j in range(num_tokens // self.bs):
                b = self.cache.get(tuple(token_ids[:(j + 1) * self.bs]))
                if b is None:
                    break
                self._hold(b)
        return super().add_sequence(sid, num_tokens, token_ids)


class PartialBlocksCached(BlockManager):
    def add_sequence(self, sid, num_tokens, token_ids=None):
        got = super().add_sequence(sid, num_tokens, token_ids)
        if token_ids is not None and num_tokens % self.bs:
            key = tuple(token_ids)
            b = self.tables[sid][-1]
            if key not in self.cache and b not in self.key_of:
                self.cache[key] = b
                self.key_of[b] = key
        return got


MUTANTS = [NoCopyOnWrite, OwnTokensKey, EvictMostRecent, FreeListQueue, ForwardRelease,
           NoTransaction, PartialBlocksCached]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda c: c.__name__)
def test_pins_catch_planted_mistakes(mutant):
    caught = []
    for pin in P.ALL_BM_PINS:
        try:
            pin(mutant)
        except Exception as e:                  # AssertionError, or a broken state
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"{mutant.__name__} passed every pin"
