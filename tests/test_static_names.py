"""Every global name a function reads is defined: a check on the source
(the symbol tables Python builds when compiling it), so that a code path the
GPU runs only on request (``bench.py --graph``, ``--ddp``) cannot fail with a
NameError there."""

import builtins
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = sorted(
    os.path.relpath(os.path.join(d, f), ROOT)
    for top in (".", "gradient_reduce_zero_amd", "oracle", "workloads", "tests")
    for d in [os.path.join(ROOT, top)]
    for f in os.listdir(d) if f.endswith(".py"))


def _undefined(path):
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    defined = {s.get_name() for s in top.get_symbols()
               if s.is_assigned() or s.is_imported() or s.is_namespace()}
    bad = []

    def walk(table):
        for sym in table.get_symbols():
            name = sym.get_name()
            if (sym.is_global() and sym.is_referenced() and name not in defined
                    and not hasattr(builtins, name) and name != "__file__"):
                bad.append(f"{table.get_name()}:{name}")
        for child in table.get_children():
            walk(child)

    for child in top.get_children():
        walk(child)
    return bad


@pytest.mark.parametrize("name", FILES)
def test_every_global_name_is_defined(name):
    assert _undefined(os.path.join(ROOT, name)) == []
