"""Static checks of bench.py's host code (no GPU): every name a function reads is defined somewhere it can
see (its own assignments and parameters, an enclosing function, the module, or the builtins). The GPU
paths of bench.py only run on the GPU, so a misspelt or stale name there would otherwise surface only in a
benchmark run."""
import ast
import builtins
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _walk_own_scope(node):
    """Nodes of `node`'s own scope: nested functions, lambdas and classes are yielded but not entered
    (their bodies bind names in scopes of their own)."""
    todo = [node]
    while todo:
        cur = todo.pop()
        yield cur
        if cur is not node and isinstance(cur, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda, ast.ClassDef)):
            continue
        todo.extend(ast.iter_child_nodes(cur))


def _bound_names(node):
    """Names bound directly in a function or module body (assignments, imports, defs, params, loops,
    comprehension targets, except-as, with-as, global/nonlocal)."""
    names = set()
    if isinstance(node, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda)):
        a = node.args
        for arg in a.posonlyargs + a.args + a.kwonlyargs:
            names.add(arg.arg)
        if a.vararg:
            names.add(a.vararg.arg)
        if a.kwarg:
            names.add(a.kwarg.arg)
    for sub in _walk_own_scope(node):
        if sub is not node and isinstance(sub, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            names.add(sub.name)
        if isinstance(sub, ast.Name) and isinstance(sub.ctx, (ast.Store, ast.Del)):
            names.add(sub.id)
        elif isinstance(sub, (ast.Import, ast.ImportFrom)):
            for al in sub.names:
                names.add((al.asname or al.name).split(".")[0])
        elif isinstance(sub, ast.ExceptHandler) and sub.name:
            names.add(sub.name)
        elif isinstance(sub, (ast.Global, ast.Nonlocal)):
            names.update(sub.names)
        elif isinstance(sub, ast.arg):
            names.add(sub.arg)
    return names


def _undefined(tree):
    missing = []
    module_names = _bound_names(tree) | set(dir(builtins)) | {"__file__", "__name__", "__doc__"}

    def visit(fn, visible):
        scope = visible | _bound_names(fn)
        for sub in _walk_own_scope(fn):
            if isinstance(sub, ast.Name) and isinstance(sub.ctx, ast.Load) and sub.id not in scope:
                missing.append((fn.name if hasattr(fn, "name") else "<lambda>", sub.id, sub.lineno))
        for inner in _walk_own_scope(fn):
            if inner is not fn and isinstance(inner, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda)):
                visit(inner, scope)

    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.AsyncFunctionDef)):
            visit(node, module_names)
    return missing


def test_bench_reads_no_undefined_name():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    assert _undefined(tree) == []


def test_checker_finds_a_planted_undefined_name():
    src = ("import time\n\ndef g():\n    c = 2\n    return c\n\n"
           "def f(a):\n    b = a + 1\n    h = lambda x: x + b\n    return {'x': round(h(b), 3), 'y': round(c, 3)}\n")
    assert [(n, name) for n, name, _ in _undefined(ast.parse(src))] == [("f", "c")]
