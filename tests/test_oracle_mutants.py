"""Planted mistakes in the oracle's prefix cache must each fail a pin.

Each mutant is the oracle's allocator module with one mistake written into
its source text (the replaced snippet must still be there, so a mutant
follows the oracle as it changes); the pins of tests/test_oracle_prefix_cache
then run against the mutant class, and at least one of them must fail.  This
shows the pins see the mistakes a plausible reading of page 3, section 04
(prefix-aware hash chain over full blocks, reference counts that protect
blocks in use, least-recently-released eviction) could make.  The mutants run
on the CPU only and never reach the HIP path.
"""

import inspect
import random
import types

import pytest

import oracle.allocator as allocator_module
import tests.test_oracle_prefix_cache as pins

# name -> [(snippet of the oracle's source, planted replacement), ...]
MUTANTS = {
    # a block's key is its own tokens instead of its whole prefix
    "non-prefix keys": [
        ("b = self.cache.get(tuple(tokens[:(i + 1) * B]))",
         "b = self.cache.get(tuple(tokens[i * B:(i + 1) * B]))"),
        ("self._enter(table[i], tuple(tokens[:(i + 1) * B]))",
         "self._enter(table[i], tuple(tokens[i * B:(i + 1) * B]))"),
        ("self._enter(table[pos // B], tuple(entry[2]))",
         "self._enter(table[pos // B], tuple(entry[2][-B:]))"),
    ],
    # a hit on a released block leaves it in the free list
    "no revival": [
        ("            if self.ref[b] == 0:\n                self.free.remove(b)\n",
         "            if self.ref[b] == 0:\n                pass\n"),
    ],
    # a block handed out again keeps its old key
    "stale keys": [
        ("            del self.cache[key]\n            self.evictions += 1\n",
         "            self.evictions += 1\n"),
    ],
    # the lookup skips a missing block and keeps matching later ones
    "no first-miss stop": [
        ("            if b is None:\n                break\n",
         "            if b is None:\n                continue\n"),
    ],
    # the partially filled last prompt block is entered too
    "partial blocks keyed": [
        ("for i in range(len(hits), n // B):", "for i in range(len(hits), -(-n // B)):"),
    ],
    # released blocks go to the head of the free list (most recently released
    # evicted first)
    "head insertion": [
        ("            if self.ref[b] == 0:\n                self.free.append(b)\n",
         "            if self.ref[b] == 0:\n                self.free.appendleft(b)\n"),
    ],
    # a hit does not take a reference on the block it maps
    "no ref on hit": [
        ("                self.free.remove(b)\n            self.ref[b] += 1\n",
         "                self.free.remove(b)\n            self.ref[b] += 0\n"),
    ],
    # a later block entered under an existing key replaces the first one
    "last key wins": [
        ("if self.prefix_caching and key not in self.cache:", "if self.prefix_caching:"),
    ],
}


def _mutant_class(replacements):
    src = inspect.getsource(allocator_module)
    for old, new in replacements:
        assert src.count(old) == 1, f"snippet not found once in the oracle: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_allocator_mutant")
    exec(compile(src, "oracle_allocator_mutant", "exec"), mod.__dict__)
    # raise the oracle's own exception class, which the pins catch by name
    mod.AllocError = allocator_module.AllocError
    return mod.BlockAllocatorModel


def _pin_calls(golden_dir):
    calls = [
        ("page example", lambda: pins.test_page_example(golden_dir)),
        ("LRU continuation", lambda: pins.test_lru_release_order_revival_and_eviction(golden_dir)),
        ("least recently released", pins.test_least_recently_released_is_evicted_first),
        ("closed form", pins.test_closed_form_shared_system_prompt),
        ("no blocks", pins.test_no_blocks_counts_revived_hits_and_changes_nothing),
        ("generated blocks", pins.test_generated_blocks_are_entered),
        ("read-only lookup", pins.test_lookup_is_read_only),
        ("brute force", pins.test_brute_force_short_op_sequences),
    ]
    calls += [(f"random stream {s}", (lambda s=s: pins.test_random_streams_keep_every_prefix_right(s)))
              for s in range(12)]
    return calls


def test_every_pin_passes_on_the_oracle(golden_dir):
    for name, call in _pin_calls(golden_dir):
        call()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, golden_dir, monkeypatch):
    monkeypatch.setattr(pins, "BlockAllocatorModel", _mutant_class(MUTANTS[name]))
    failed = []
    for pin, call in _pin_calls(golden_dir):
        try:
            call()
        except (Exception, pytest.fail.Exception) as e:  # a failed check or a provoked error
            failed.append((pin, type(e).__name__))
    print(name, "fails", failed)
    assert failed, f"mutant '{name}' passes every prefix-cache pin"
