"""Planted mistakes in the oracle's block allocator (outside the prefix cache,
which tests/test_oracle_mutants.py covers) must each fail a pin.

Each mutant is the oracle's allocator module with one mistake written into its
source text (the replaced snippet must still be there once).  The pins of
tests/test_oracle_allocator and tests/test_oracle_swap then run against the
mutant class, and at least one must fail.  The mistakes are ones a reading of
the pages' allocator could plausibly make: a block taken when a token fills
its block instead of when the next one crosses into a new block, a sequence
released first block first, a fork that takes no references, a shared
partial block written in place, a copy-on-write that leaves the old block's
count, a step whose block count forgets the copies, a wrong in-block slot, and
a swap that leaves the device counts behind.  CPU only.
"""

import inspect
import types

import pytest

import oracle.allocator as allocator_module
import tests.test_oracle_allocator as allocator_pins
import tests.test_oracle_swap as swap_pins

PIN_MODULES = [allocator_pins, swap_pins]

MUTANTS = {
    "eager allocation when a block fills": [
        ("        if pos % B == 0:\n            # The new token crosses into a block not yet mapped",
         "        if pos % B == 0 and pos // B >= len(table):\n            # The new token crosses into a block not yet mapped"),
        ("        slot = self._slot(table, pos)\n        entry = self.seqs[seq]\n",
         "        slot = self._slot(table, pos)\n        if (pos + 1) % B == 0 and self.free:\n"
         "            table.append(self._take())\n        entry = self.seqs[seq]\n"),
    ],
    "release first block first": [
        ("        table = self.seqs.pop(seq)[0]\n        for b in reversed(table):",
         "        table = self.seqs.pop(seq)[0]\n        for b in table:"),
    ],
    "fork takes no references": [
        ("        for b in table:\n            self.ref[b] += 1\n        self.seqs[child]",
         "        for b in table:\n            self.ref[b] += 0\n        self.seqs[child]"),
    ],
    "shared partial block written in place": [
        ("            if self.ref[last] > 1:\n                # Divergent write",
         "            if self.ref[last] > 99:\n                # Divergent write"),
    ],
    "copy-on-write keeps the old block's count": [
        ("                self.ref[last] -= 1\n                table[pos // B] = fresh",
         "                table[pos // B] = fresh"),
    ],
    "step's block count forgets the copies": [
        ("            elif ref[table[pos // B]] > 1:\n                needed += 1",
         "            elif ref[table[pos // B]] > 1:\n                needed += 0"),
    ],
    "slot offset shifted": [
        ("        return table[pos // B] * B + pos % B",
         "        return table[pos // B] * B + (pos + 1) % B"),
    ],
    "swap leaves the source counts": [
        ("            src_ref[b] = 0\n            src_release(b)",
         "            src_release(b)"),
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


def _pins(golden_dir):
    calls = []
    for m in PIN_MODULES:
        for name, fn in sorted(vars(m).items()):
            if not name.startswith("test_") or not callable(fn):
                continue
            params = inspect.signature(fn).parameters
            extra = {"golden_dir": golden_dir} if "golden_dir" in params else {}
            marks = [mk for mk in getattr(fn, "pytestmark", []) if mk.name == "parametrize"]
            if marks:
                argname, values = marks[0].args[0], marks[0].args[1]
                calls += [(f"{m.__name__}.{name}[{v}]",
                           (lambda fn=fn, a=argname, v=v, e=extra: fn(**{a: v}, **e)))
                          for v in values]
            else:
                calls.append((f"{m.__name__}.{name}", (lambda fn=fn, e=extra: fn(**e))))
    return calls


def test_every_pin_passes_on_the_oracle(golden_dir):
    for name, call in _pins(golden_dir):
        call()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, golden_dir, monkeypatch):
    cls = _mutant_class(MUTANTS[name])
    for pins in PIN_MODULES:
        if hasattr(pins, "BlockAllocatorModel"):
            monkeypatch.setattr(pins, "BlockAllocatorModel", cls)
    failed = []
    for pin, call in _pins(golden_dir):
        try:
            call()
        except (Exception, pytest.fail.Exception) as e:  # a failed check or a provoked error
            failed.append((pin, type(e).__name__))
    print(name, "fails", failed[:5], f"({len(failed)} pins)")
    assert failed, f"mutant '{name}' passes every allocator pin"
