"""The C oracle and the corpus generator under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, gcc).

oracle/sanitize_check.c drives the brute-force pins through the C entry
points (literal == chunk-multiset training on every short string over a
five-byte alphabet, and on small corpora of every recipe: encoding the
training text gives the training tokens, longest-match tokens cover the
text); any invalid access, use after free, overflow or undefined operation
aborts the run with a sanitizer report."""
import subprocess

import corpus
import oracle


def test_oracle_and_generator_pins_under_asan_and_ubsan(tmp_path):
    exe = corpus.build(force=True, sanitize=True, out_dir=str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok:"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_sanitizer_flags_are_on():
    assert "-fsanitize=address,undefined" in oracle.SANITIZE_FLAGS
    assert "-fno-sanitize-recover=all" in oracle.SANITIZE_FLAGS
