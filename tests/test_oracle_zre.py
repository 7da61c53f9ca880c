"""Pins of the oracle's zero-run encoding (3LC page, "Proposed method",
item 3: a run-length variant for runs of the zero byte; codes 243..255 stand
for runs of 2..14 zero bytes).

The decoder is checked on its own (it is a per-byte expansion), and the
encoder against: brute force over every string of length <= 12 on the
alphabet {121, 0, 242}, the closed-form length, the hand-worked examples,
runs of every length 1..200, long random strings, and the greedy canonical
form (chunks of 14 from the run start)."""
import os

import numpy as np
import pytest

import oracle

Z = 121
SEP = 7  # never produced by encoding strings over {121, 0, 242}


def closed_form_len(b: np.ndarray) -> int:
    """L = (#bytes != 121) + sum over maximal runs of 121 of ceil(r/14)."""
    L = int(np.count_nonzero(b != Z))
    r = 0
    for v in b.tolist() + [None]:
        if v == Z:
            r += 1
        else:
            L += -(-r // 14)
            r = 0
    return L


def run_code(r: int) -> list[int]:
    """Stream bytes for an isolated run of r zero bytes: 14-chunks from the start."""
    out = [255] * (r // 14)
    m = r % 14
    if m == 1:
        out.append(121)
    elif m >= 2:
        out.append(241 + m)
    return out


def expand(runs):
    return np.array([v for v, k in runs for _ in range(k)], dtype=np.uint8)


def test_decoder_is_per_byte_expansion():
    # each byte < 243 decodes to itself, each code c >= 243 to c-241 zero bytes
    for c in range(256):
        want = [c] if c < 243 else [Z] * (c - 241)
        got = oracle.zre_decode(np.array([c], dtype=np.uint8), len(want))
        assert got.tolist() == want


def strings_of_length(l: int) -> np.ndarray:
    alphabet = np.array([Z, 0, 242], dtype=np.uint8)
    idx = np.arange(3 ** l, dtype=np.int64)
    digits = np.stack([(idx // 3 ** j) % 3 for j in range(l)], axis=1) if l else np.zeros((1, 0), np.int64)
    return alphabet[digits]


def test_bruteforce_small_strings_encoded_one_by_one():
    # every string of length <= 7 on its own: round trip and closed-form length
    for l in range(0, 8):
        for row in strings_of_length(l):
            enc = oracle.zre_encode(row)
            assert enc.size == closed_form_len(row) <= max(row.size, 0)
            assert np.array_equal(oracle.zre_decode(enc, row.size), row)


def test_bruteforce_all_strings_up_to_12():
    # 797,161 strings, encoded in one call with a separator literal after each
    # string.  The decoder is a per-byte map, so decode(encode(S)) == S and the
    # separators splitting the stream into one piece per string prove that
    # every piece decodes to its own string; the encoding of strings of length
    # <= 7 alone is pinned by the previous test.
    parts, lengths = [], []
    for l in range(0, 13):
        rows = strings_of_length(l)
        block = np.full((rows.shape[0], l + 1), SEP, dtype=np.uint8)
        block[:, :l] = rows
        parts.append(block.ravel())
        # closed form for runs shorter than 14: one code per run
        nz = np.count_nonzero(rows != Z, axis=1)
        starts = (rows == Z) & np.concatenate([np.ones((rows.shape[0], 1), bool), rows[:, :-1] != Z], axis=1) \
            if l else np.zeros((1, 0), bool)
        lengths.append(nz + starts.sum(axis=1))
    S = np.concatenate(parts)
    want_len = np.concatenate(lengths)
    assert want_len.size == (3 ** 13 - 1) // 2
    enc = oracle.zre_encode(S)
    assert np.array_equal(oracle.zre_decode(enc, S.size), S)
    cuts = np.flatnonzero(enc == SEP)
    assert cuts.size == want_len.size
    piece_len = np.diff(np.concatenate([[-1], cuts])) - 1
    assert np.array_equal(piece_len, want_len)
    assert np.all(piece_len <= np.concatenate([np.full(3 ** l, l) for l in range(13)]))


def test_golden_zre(golden):
    for case in golden["zre"]:
        b = expand(case["bytes_runs"])
        enc = oracle.zre_encode(b)
        assert enc.tolist() == case["stream"], case["id"]
        assert np.array_equal(oracle.zre_decode(enc, b.size), b)


def test_runs_of_every_length():
    for r in range(1, 201):
        b = np.full(r, Z, dtype=np.uint8)
        enc = oracle.zre_encode(b)
        assert enc.tolist() == run_code(r)
        assert enc.size == -(-r // 14)
        # the same run between literals
        b2 = np.concatenate([[5], b, [9]]).astype(np.uint8)
        assert oracle.zre_encode(b2).tolist() == [5] + run_code(r) + [9]


def test_max_ratio_is_14():
    for B in (14, 140, 14_000, 1_000_003):
        b = np.full(B, Z, dtype=np.uint8)
        assert oracle.zre_encode(b).size == -(-B // 14)


def test_no_zero_bytes_is_identity():
    rng = np.random.default_rng(0)
    b = rng.integers(0, 243, 5000).astype(np.uint8)
    b[b == Z] = 0
    assert np.array_equal(oracle.zre_encode(b), b)


@pytest.mark.parametrize("seed", range(6))
def test_random_long_strings(seed):
    rng = np.random.default_rng(100 + seed)
    # runs with lengths spanning many 14-chunks, separated by literals
    chunks = []
    while sum(map(len, chunks)) < 10_000:
        r = int(rng.choice([0, 1, 2, 13, 14, 15, 27, 28, 29, int(rng.integers(1, 600))]))
        chunks.append([Z] * r)
        chunks.append(rng.integers(0, 243, int(rng.integers(1, 4))).tolist())
    b = np.array([v for c in chunks for v in c], dtype=np.uint8)
    enc = oracle.zre_encode(b)
    assert enc.size == closed_form_len(b) <= b.size
    assert np.array_equal(oracle.zre_decode(enc, b.size), b)
    check_canonical(enc)


def check_canonical(enc: np.ndarray):
    """Greedy split from the run start: inside one run the stream is
    255...255 then at most one remainder code, so a remainder code (243..254)
    is never followed by a run code, and 255 is never preceded by a remainder
    code.  (An end-anchored split would put a remainder first.)"""
    e = enc.tolist()
    for a, b in zip(e, e[1:]):
        if 243 <= a <= 254:
            assert b < 243 and b != Z
        if a == Z:
            assert b < 243


def test_decoder_rejects_malformed_streams():
    b = expand([[Z, 20], [3, 1], [Z, 5]])
    enc = oracle.zre_encode(b)
    with pytest.raises(oracle.OracleError):
        oracle.zre_decode(enc[:-1], b.size)            # truncated
    with pytest.raises(oracle.OracleError):
        oracle.zre_decode(np.concatenate([enc, [3]]).astype(np.uint8), b.size)  # extra byte
    with pytest.raises(oracle.OracleError):
        oracle.zre_decode(np.array([255], dtype=np.uint8), 13)  # run overruns B
    with pytest.raises(oracle.OracleError):
        oracle.zre_decode(np.array([], dtype=np.uint8), 1)      # empty stream, B > 0
    assert oracle.zre_decode(np.array([], dtype=np.uint8), 0).size == 0


@pytest.mark.skipif(os.environ.get("TLC_SKIP_SANITIZE") == "1", reason="disabled")
def test_oracle_under_asan_ubsan(tmp_path):
    """Host sanitizers on the oracle: build it with ASan+UBSan and drive the
    codec through a small C program (host code only)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    here = os.path.dirname(oracle.__file__)
    prog = tmp_path / "drive.c"
    prog.write_text(r'''
#include "tlc_oracle.h"
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
int main(void) {
  for (uint64_t n = 1; n < 300; n += 7) {
    float* x = malloc(n * sizeof(float)); float* e = calloc(n, sizeof(float));
    float* y = malloc(n * sizeof(float));
    uint64_t B = tlco_quartic_len(n); uint8_t* s = malloc(B);
    for (uint64_t i = 0; i < n; ++i) x[i] = (float)((int)(i * 2654435761u % 1000) - 500) * 1e-3f;
    uint64_t L; float M;
    if (tlco_compress(x, e, n, 1.5f, s, B, &L, &M)) return 1;
    if (tlco_decompress(s, L, M, n, 1.5f, y)) return 2;
    if (L > 0 && tlco_decompress(s, L - 1, M, n, 1.5f, y) != TLCO_ERR_CORRUPT) return 3;
    free(x); free(e); free(y); free(s);
  }
  puts("ok"); return 0;
}
''')
    exe = tmp_path / "drive"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", here, str(prog), os.path.join(here, "tlc_oracle.c"),
                    "-o", str(exe), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
