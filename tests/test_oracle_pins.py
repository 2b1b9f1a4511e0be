"""CPU tests: the oracle against its pins, and mutated oracles against the same pins."""
import os
import subprocess
import sys

import pytest

import oracle
from oracle_pins import PINS

# Plausible mistakes, each planted into a copy of oracle.c: (name, original text, mutated text).
MUTATIONS = [
    ("scale dropped", "logits[cnt] = scale * dot;", "logits[cnt] = dot;"),
    ("lse sign", "lse[(size_t)b * Hq + h] = m + log(z);", "lse[(size_t)b * Hq + h] = m - log(z);"),
    ("gqa interleaved", "int kvh = h / G;\n    int64_t cnt = 0;", "int kvh = h % Hkv;\n    int64_t cnt = 0;"),
    ("window off by one", "return t < sinks || t >= L - window;", "return t < sinks || t > L - window;"),
    ("sinks ignored", "return t < sinks || t >= L - window;", "return t >= L - window;"),
    ("K chunk strides swapped", "(size_t)(x / (4 * E)) * 64 + (size_t)((x / E) % 4) * 16 + tau",
     "(size_t)(x / (4 * E)) * 16 + (size_t)((x / E) % 4) * 64 + tau"),
    ("V token split transposed", "int n = x / 16, c = x % 16, j = tau / 4, i = tau % 4;",
     "int n = x / 16, c = x % 16, j = tau % 4, i = tau / 4;"),
    ("V read from K pool", "o[x] += w * load_cache(vpool, num_blocks, (size_t)blk, kvh, (int)(t % P), x, Hkv, P, d, dt, 1);",
     "o[x] += w * load_cache(kpool, num_blocks, (size_t)blk, kvh, (int)(t % P), x, Hkv, P, d, dt, 0);"),
    ("normaliser not shifted", "for (int64_t k = 0; k < cnt; ++k) z += exp(logits[k] - m);",
     "for (int64_t k = 0; k < cnt; ++k) z += exp(logits[k]);"),
    ("block index uses offset", "int64_t blk = bt_row[t / P];", "int64_t blk = bt_row[t % P];"),
    ("page-list partitions ranked over attended units", "                if (pages) {\n                    int e = page_entry",
     "                if (0) {\n                    int e = page_entry"),
    ("page entry not scaled by units per page", "u = (int64_t)e * (P / 16) + (t % P) / 16;", "u = (int64_t)e + (t % P) / 16;"),
    ("combine weight inverted", "double w = exp(pm[s] - M);", "double w = exp(M - pm[s]);"),
    ("fp16 exponent bias", "v = ldexp((double)(f | 0x400), e - 25);", "v = ldexp((double)(f | 0x400), e - 24);"),
    ("bf16 wrong half", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("KV formula missing K/V factor", "return 2ull * (uint64_t)batch", "return 1ull * (uint64_t)batch"),
    ("page test uses offset", "if (pages[k] >= 0 && pages[k] == t / P) return 1;",
     "if (pages[k] >= 0 && pages[k] == t % P) return 1;"),
    ("min instead of max", "for (int64_t k = 1; k < cnt; ++k) if (logits[k] > m) m = logits[k];",
     "for (int64_t k = 1; k < cnt; ++k) if (logits[k] < m) m = logits[k];"),
    ("append skips last head", "for (int h = 0; h < Hkv; ++h)\n            for (int x = 0; x < d; ++x) {\n                size_t src",
     "for (int h = 0; h + 1 < Hkv; ++h)\n            for (int x = 0; x < d; ++x) {\n                size_t src"),
    ("paged rounding dropped", "if (block_size > 0) seq =", "if (block_size < 0) seq ="),
    ("score not normalised", "row[e] += exp(logits[k] - m) / z;", "row[e] += exp(logits[k] - m);"),
    ("score row per head, not per group", "double* row = score + ((size_t)b * Hkv + h / G) * (size_t)stride;",
     "double* row = score + ((size_t)b * Hkv + h % Hkv) * (size_t)stride;"),
    ("score overwritten, not added", "row[e] += exp(logits[k] - m) / z;", "row[e] = exp(logits[k] - m) / z;"),
    ("score entry by token, not block", "int64_t e = toks[k] / block;", "int64_t e = toks[k] / (block > 1 ? block - 1 : 1);"),
    ("page ties to the higher id", "if (best < 0 || w[p] > w[best]) best = p;", "if (best < 0 || w[p] >= w[best]) best = p;"),
    ("page weights in double", "float acc = 0.0f;", "double acc = 0.0;"),
    ("newest page not forced", "for (int64_t p = first_recent; p < n; ++p) row[cnt++] = (int32_t)p;", ";"),
    ("k pages besides the newest", "int64_t want = k - recent;", "int64_t want = k;"),
    ("int8 rounding truncates", "float r = rintf(x[i] * inv);", "float r = truncf(x[i] * inv);"),
    ("int8 scale not applied", "return (double)q * (double)sc;", "return (double)q;"),
    ("int8 scale per tile, not per row", "memcpy(&sc, (const char*)pool + plane + (((size_t)blk * Hkv + h) * P + t) * 4, 4);",
     "memcpy(&sc, (const char*)pool + plane + (((size_t)blk * Hkv + h) * P) * 4, 4);"),
    ("int8 amax from the first element", "if (a > amax) amax = a;", "if (i == 0) amax = a;"),
    ("ring size ignores the page offset", "int touched = (o + window + P - 1) / P;",
     "int touched = (window + P - 1) / P;"),
    ("ring column drops the sink offset", "return sp + (page - sp) % ring_pages;",
     "return (page - sp) % ring_pages;"),
    ("sink pages rounded down", "return sinks > 0 ? ((int64_t)sinks + P - 1) / P : 0;", "return sinks / P;"),
    ("window blocks counted per page", "if (!used[c]) { used[c] = 1; ++n; }", "{ used[c] = 1; ++n; }"),
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.default())


@pytest.mark.parametrize("name,orig,mut", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, orig, mut):
    src = open(oracle.SOURCE).read()
    assert src.count(orig) >= 1, f"mutation anchor not found: {name}"
    path = tmp_path / "oracle_mut.c"
    path.write_text(src.replace(orig, mut))
    so = oracle.compile_oracle(str(path), str(tmp_path / "liboracle_mut.so"))
    # A mutated oracle may write out of bounds, so its pins run in a child process; a crash
    # there also counts as the mistake being caught.
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([os.path.dirname(here), here]))
    r = subprocess.run([sys.executable, os.path.join(here, "oracle_pins.py"), so], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin catches the planted mistake: {name}"
