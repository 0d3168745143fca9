"""Static check of the committed scripts that only a GPU run executes end to
end (bench.py, __graft_entry__.py): every name a function reads is bound
somewhere in that function (its arguments, assignments, imports, nested
functions, comprehensions, handlers), at module level, or is a builtin.
It catches a name left behind by a refactor before a GPU run does."""
import ast
import builtins
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _module_names(tree):
    names = set()
    for n in tree.body:
        if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            names.add(n.name)
        elif isinstance(n, (ast.Assign, ast.AnnAssign, ast.AugAssign)):
            targets = n.targets if isinstance(n, ast.Assign) else [n.target]
            for t in targets:
                names.update(x.id for x in ast.walk(t) if isinstance(x, ast.Name))
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            names.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, (ast.If, ast.Try, ast.With)):
            for x in ast.walk(n):
                if isinstance(x, ast.Name) and isinstance(x.ctx, ast.Store):
                    names.add(x.id)
                elif isinstance(x, (ast.Import, ast.ImportFrom)):
                    names.update((a.asname or a.name).split(".")[0] for a in x.names)
    return names


def _unbound(fn, module_names):
    bound = set()
    for x in ast.walk(fn):
        if isinstance(x, ast.arg):
            bound.add(x.arg)
        elif isinstance(x, ast.Name) and isinstance(x.ctx, (ast.Store, ast.Del)):
            bound.add(x.id)
        elif isinstance(x, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            bound.add(x.name)
        elif isinstance(x, (ast.Import, ast.ImportFrom)):
            bound.update((a.asname or a.name).split(".")[0] for a in x.names)
        elif isinstance(x, ast.ExceptHandler) and x.name:
            bound.add(x.name)
        elif isinstance(x, (ast.Global, ast.Nonlocal)):
            bound.update(x.names)
    used = {x.id for x in ast.walk(fn) if isinstance(x, ast.Name) and isinstance(x.ctx, ast.Load)}
    return sorted(used - bound - module_names - set(dir(builtins)))


@pytest.mark.parametrize("script", ["bench.py", "__graft_entry__.py"])
def test_functions_read_only_bound_names(script):
    tree = ast.parse(open(os.path.join(ROOT, script)).read(), script)
    mod = _module_names(tree)
    # top-level functions and methods; a nested function is checked as part
    # of the function that encloses it (its closure names are bound there)
    fns = [n for n in tree.body if isinstance(n, ast.FunctionDef)]
    fns += [m for c in tree.body if isinstance(c, ast.ClassDef) for m in c.body
            if isinstance(m, ast.FunctionDef)]
    bad = {}
    for node in fns:
        u = _unbound(node, mod)
        if u:
            bad[node.name] = u
    assert not bad, f"{script}: names read but never bound: {bad}"
