"""Serialized-launch debug mode gives the same bits as normal launches.

A child process runs the seeded random configurations of
tests/test_gpu_random_configs.py (every mask family; the backward on interval and
bitmap masks; the one-pass, block-major and split forms of the selected-key path)
and prints a hash of every output.  It runs twice: as is, and with
AMD_SERIALIZE_KERNEL=3 and HIP_LAUNCH_BLOCKING=1, where every launch waits for
the previous one and returns only when it has finished.  All of the library's
work is ordered on the caller's stream, so the two runs must agree bit for
bit; a difference would point at work that depends on launch timing (a
missing wait, host code reading device memory too early).
"""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SEEDS = 24

CHILD = r"""
import hashlib, json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import mask_aware_block_amd as fm
import synth
from tests.helpers import to_device
from tests.test_gpu_random_configs import _case

def h(t):
    return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()[:16]

out = {}
for seed in range(int(sys.argv[2])):
    w, spec, rng = _case(seed)
    q, k, v = to_device(w, synth.draw_qkv(w))
    enc = fm.encode(spec)
    res = []
    if enc.kind == fm.ENC_SELECTED:
        res += fm.attn_fwd(q, k, v, enc, None, scale=w["scale"])
        res += fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"])
        res += fm.attn_fwd_split(q, k, v, enc, splits=3, scale=w["scale"])
    else:
        tiles = fm.classify(enc, 128, 64)
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        res += [o, lse]
        if enc.kind in (fm.ENC_INTERVALS, fm.ENC_BITMAP):
            do = torch.from_numpy(synth.draw_dout(w).view(np.int16)).view(torch.bfloat16).cuda()
            res += fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    out[seed] = [h(x) for x in res]
    print("seed", seed, spec["family"], flush=True, file=sys.stderr)
print(json.dumps(out))
"""


def _run(extra_env):
    env = dict(os.environ, **extra_env)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(SEEDS)], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=240)
    assert r.returncode == 0, f"child failed ({extra_env}):\n{r.stderr[-4000:]}"
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_serialized_launches_give_the_same_bits():
    normal = _run({})
    serial = _run({"AMD_SERIALIZE_KERNEL": "3", "HIP_LAUNCH_BLOCKING": "1"})
    assert len(normal) == SEEDS
    diff = {s: (normal[s], serial.get(s)) for s in normal if normal[s] != serial.get(s)}
    assert not diff, f"outputs differ under serialized launches: {diff}"
