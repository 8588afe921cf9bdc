"""Planted mistakes in the oracle's attention and cache operations must each
fail a pin.

Each mutant is one of the oracle's modules with a mistake written into its
source text (the replaced snippet must still be there once, so a mutant
follows the oracle as it changes).  The pins of tests/test_oracle_attention,
tests/test_oracle_prefill and tests/test_oracle_cache_ops then run against
the mutant's functions, and at least one of them must fail.  The mistakes are
the ones a reading of the pages' attention and write could plausibly make: a
dropped scale, the wrong KV head for a query head, a context one token short,
a wrong in-block offset or block index, a missing normalisation, a causal
mask that lets the next token in, new tokens placed at the wrong positions,
the first query reused, a wrong bf16 widening, a write to the wrong offset,
and a copy that reads blocks already overwritten.  The mutants run on the
CPU only and never reach the HIP path.
"""

import inspect
import types

import pytest

import oracle.attention as attention_module
import oracle.cache_ops as cache_ops_module
import tests.test_oracle_attention as attention_pins
import tests.test_oracle_cache_ops as cache_ops_pins
import tests.test_oracle_prefill as prefill_pins

PIN_MODULES = [attention_pins, prefill_pins, cache_ops_pins]

# the decode's gather: the V line carries a comment the prefill's lacks
DECODE_GATHER = (
    "        blocks = [int(block_tables[s][t // B]) for t in range(n)]\n"
    "        offsets = [t % B for t in range(n)]\n"
    "        gathered = {}  # KV head -> its gathered (K, V), shared by the head's G query heads\n"
    "        for h in head_list:\n"
    "            g = h // G\n"
    "            if g not in gathered:\n"
    "                gathered[g] = (to_f64(k_cache[blocks, g, offsets, :], dtype),   # [n, D]\n"
    "                               to_f64(v_cache[blocks, g, offsets, :], dtype))   # [n, D]\n")
PREFILL_HEAD = (
    "            g = h // G\n"
    "            if g not in gathered:\n"
    "                gathered[g] = (to_f64(k_cache[blocks, g, offsets, :], dtype),   # [n, D]\n"
    "                               to_f64(v_cache[blocks, g, offsets, :], dtype))\n")


def _swap(text, old, new):
    return [(text, text.replace(old, new))]


# name -> (module, [(snippet of the module's source, planted replacement), ...])
MUTANTS = {
    "decode: scale dropped": (attention_module, [
        ("logits = scale * (K @ qh)", "logits = (K @ qh)")]),
    "decode: query head h reads KV head h % Hkv": (attention_module, _swap(
        DECODE_GATHER, "g = h // G", "g = h % Hkv")),
    "decode: context one token short": (attention_module, _swap(
        DECODE_GATHER, "for t in range(n)]", "for t in range(n - 1)]")),
    "decode: in-block offset shifted": (attention_module, _swap(
        DECODE_GATHER, "offsets = [t % B for", "offsets = [(t + 1) % B for")),
    "decode: block index t % B": (attention_module, _swap(
        DECODE_GATHER, "block_tables[s][t // B]", "block_tables[s][t % B]")),
    "decode: no normalisation": (attention_module, [
        ("out[s, h, :] = (w @ V) / w.sum()", "out[s, h, :] = (w @ V)")]),
    "prefill: mask lets the next token in": (attention_module, [
        ("logits = scale * (K[: p + 1] @ qh)", "logits = scale * (K[: p + 2] @ qh)"),
        ("(w @ V[: p + 1])", "(w @ V[: p + 2])")]),
    "prefill: new tokens one position early": (attention_module, [
        ("        first = n - n_new\n", "        first = max(0, n - n_new - 1)\n")]),
    "prefill: query head h reads KV head h % Hkv": (attention_module, _swap(
        PREFILL_HEAD, "g = h // G", "g = h % Hkv")),
    "prefill: first new token's query for every row": (attention_module, [
        ("qh = to_f64(q[qsl[s] + j, h, :], dtype)", "qh = to_f64(q[qsl[s], h, :], dtype)")]),
    "bf16 widened by the wrong shift": (attention_module, [
        ("(x.astype(np.uint32) << np.uint32(16))", "(x.astype(np.uint32) << np.uint32(15))")]),
    "write: offset and block swapped": (cache_ops_module, [
        ("    block = slots[keep] // B\n    offset = slots[keep] % B\n",
         "    block = slots[keep] % B\n    offset = slots[keep] // B % B\n")]),
    "write: slots past the pool kept": (cache_ops_module, [
        ("keep = np.nonzero((slots >= 0) & (slots < num_blocks * B))[0]",
         "keep = np.nonzero(slots >= -1)[0]")]),
    "copy: reads blocks already overwritten": (cache_ops_module, [
        ("        kc[int(d)] = src_k[int(s)]\n        vc[int(d)] = src_v[int(s)]\n",
         "        kc[int(d)] = kc[int(s)]\n        vc[int(d)] = vc[int(s)]\n")]),
}


def _mutant(module, replacements):
    src = inspect.getsource(module)
    for old, new in replacements:
        assert src.count(old) == 1, f"snippet not found once in {module.__name__}: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType(module.__name__ + "_mutant")
    exec(compile(src, module.__name__ + "_mutant", "exec"), mod.__dict__)
    return mod


def _pins():
    """Every pin of the three modules, parametrized ones once per case."""
    calls = []
    for m in PIN_MODULES:
        for name, fn in sorted(vars(m).items()):
            if not name.startswith("test_") or not callable(fn):
                continue
            marks = [mk for mk in getattr(fn, "pytestmark", []) if mk.name == "parametrize"]
            if marks:
                argname, values = marks[0].args[0], marks[0].args[1]
                calls += [(f"{m.__name__}.{name}[{i}]", (lambda fn=fn, a=argname, v=v: fn(**{a: v})))
                          for i, v in enumerate(values)]
            else:
                calls.append((f"{m.__name__}.{name}", fn))
    return calls


def test_every_pin_passes_on_the_oracle():
    for name, call in _pins():
        call()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, monkeypatch):
    module, replacements = MUTANTS[name]
    mod = _mutant(module, replacements)
    for pins in PIN_MODULES:
        for fn_name in ("paged_attention_decode", "paged_attention_prefill", "paged_kv_write",
                        "copy_blocks"):
            if hasattr(pins, fn_name) and hasattr(mod, fn_name):
                monkeypatch.setattr(pins, fn_name, getattr(mod, fn_name))
    failed = []
    for pin, call in _pins():
        try:
            call()
        except (Exception, pytest.fail.Exception) as e:  # a failed check or a provoked error
            failed.append((pin, type(e).__name__))
    print(name, "fails", failed[:6], f"({len(failed)} pins)")
    assert failed, f"mutant '{name}' passes every attention and cache-op pin"
