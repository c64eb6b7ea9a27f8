"""Command-line contract of bench.py that needs no GPU: a request for more
than one GPU ends at once with a message and a non-zero status."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.lstrip().startswith("{")  # no JSON line for an unsupported run


def test_counter_summaries_key_on_code_not_comments():
    """The committed counter traffic applies while the kernels' code is the one
    it was taken with: comments and blank lines do not change the digest,
    a change of code does; string literals are code."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    a = 'int f(int x) {  // doubles x\n  /* a block\n     comment */ return 2 * x;\n}\nconst char* s = "// kept";\n'
    b = 'int f(int x) {\n\n  return 2 * x;   \n}\nconst char* s = "// kept";  /* note */\n'
    c = 'int f(int x) {\n  return 3 * x;\n}\nconst char* s = "// kept";\n'
    assert bench.source_code(a) == bench.source_code(b)
    assert bench.source_code(a) != bench.source_code(c)
    assert '"// kept"' in bench.source_code(a)
    assert len(bench.kernel_source_sha()) == 16
