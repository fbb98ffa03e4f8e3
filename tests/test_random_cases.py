"""Seeded random decode configurations on the GPU against the oracle: batch,
query length, head count, page size, ragged lengths (empty requests
included), pool type and k_scale, split mode -- drawn per seed, so that
combinations the hand-picked cases miss are covered too."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle
from oracle import ragged as RG
import oracle_pins as P
from mla_synth import ragged
import gpu_util as G
from test_ragged import run_ragged


def _draw(seed):
    r = np.random.default_rng(7000 + seed)
    B = int(r.integers(1, 13))
    q_len = int(r.integers(1, 5))
    H = int(r.choice([1, 8, 16, 40, 64, 128]))
    Pg = int(r.choice([32, 64]))
    lens = r.integers(0, 700, size=B)
    lens[r.random(B) < 0.15] = 0
    kv = "fp8" if r.random() < 0.35 else "bf16"
    k_scale = float(r.choice([0.5, 0.25, 1.5])) if kv == "fp8" else None
    mode = r.choice(["auto", "forced", "units"])
    kw = {"auto": {}, "forced": {"num_splits": int(r.integers(1, 10))},
          "units": {"min_work_units": int(r.integers(1, 64))}}[mode]
    inp = P.small(kv=kv, q_len=q_len, heads=H, page_size=Pg, lens=tuple(int(x) for x in lens), seed=7000 + seed,
                  k_scale=k_scale)
    return inp, kw, r


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(seed):
    inp, kw, _ = _draw(seed)
    o, l = G.run(inp, **kw)
    ro, rl = oracle.default().decode(inp)
    G.compare(o, l, ro, rl, fp8=inp.kv_fp8, what=f"seed {seed}: B={inp.batch} q={inp.q_len} H={inp.heads} "
                                                  f"P={inp.page_size} fp8={inp.kv_fp8} {kw}")


@pytest.mark.parametrize("seed", range(8))
def test_random_ragged(seed):
    inp, kw, r = _draw(100 + seed)
    q_lens = r.integers(0, inp.q_len + 1, size=inp.batch)
    rg = ragged(inp, q_lens=q_lens)
    o, l = run_ragged(rg, **kw)
    ro, rl = RG.decode(oracle.default(), rg)
    G.compare(o, l, ro, rl, fp8=inp.kv_fp8, what=f"ragged seed {seed}: q_lens={list(q_lens)} {kw}")
