"""GPU parity on peaked attention: the cases that drive the online softmax
of the split partial kernel (an FA2-style running max, sum and output per
split, page "perf(gfx1100): speed up long-context DFlash verify 13.4% with FA2
split-KV and retain HipGraph/Redline PM4", Summary) through its rescale path
with finite earlier state, at the headline shape (B 16, 24 query heads over 4
KV heads, head_dim 256, 8-bit KV) and 8,192 / 32,768 tokens:

- Q scaled by 4 and 16: score deviations of 4 and 16 nats, a few keys carry
  each row, and every K rounding shows in the weights;
- scores that rise along the context (24 and 8 base-2 units per 64-key tile),
  so the running max is raised on every tile or every other tile while the
  earlier keys still weigh in;
- one dominant key near the end (in the last split of every split count).

Each case runs at S = 1 (direct), 8 and the plan's split count, with fp32,
fp16 and bf16 output, against the fp64 oracle at the gate of the other parity
tests (bf16: also the fp32 twin and bf16 == RNE(fp32)).
"""

import numpy as np
import pytest

import oracle
import synthetic as S

from .gpu_util import check_bf16_twin, check_parity, ensure_lib, run_gpu, say

pytestmark = pytest.mark.gpu

CASES = {
    "gain4": lambda ctx: S.peaked(ctx, 4.0),
    "gain16": lambda ctx: S.peaked(ctx, 16.0),
    "rise24": lambda ctx: S.rising_max(ctx, 0.375),
    "rise8": lambda ctx: S.rising_max(ctx, 0.125),
    "late_dominant": lambda ctx: S.late_dominant(ctx),
}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


_cache = {}


def wl(name, ctx):
    key = (name, ctx)
    if key not in _cache:
        say(f"[gen] {name} ctx={ctx}")
        w = CASES[name](ctx)
        say(f"[oracle] {w.name}")
        _cache[key] = (w,) + tuple(oracle.attention(w))
    return _cache[key]


@pytest.mark.parametrize("ctx", [8192, 32768])
@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("S_", [1, 8, 0])
def test_peaked(name, ctx, S_):
    w, o, l = wl(name, ctx)
    say(f"[case] {name} ctx={ctx} S={S_}")
    f32, lse, flags, info = run_gpu(w, S_, "f32")
    assert flags == 0
    check_parity(f32, o, "f32", f"{name} ctx={ctx} S={S_ or info.num_splits} f32")
    assert np.abs(lse - l).max() <= 1e-4 * max(1.0, np.abs(l).max())
    f16 = run_gpu(w, S_, "f16")[0]
    check_parity(f16, o, "f16", f"{name} ctx={ctx} S={S_ or info.num_splits} f16")
    b16 = run_gpu(w, S_, "bf16")[0]
    check_bf16_twin(b16, f32, o, f"{name} ctx={ctx} S={S_ or info.num_splits} bf16")
