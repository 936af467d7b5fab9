"""The optional launch log: MI355ATTN_LOG=1 makes every launch print one line to
stderr; without it the library prints nothing."""
import os
import subprocess
import sys

import pytest
import torch

import exact_attention_46_amd as ea

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import torch
import exact_attention_46_amd as ea
q = torch.randn(1, 2, 128, 64, device="cuda").half()
o, lse = ea.fwd(q, q, q, causal=True)
dq, dk, dv = ea.bwd(q, q, q, o, lse, torch.ones_like(q), causal=True)
qd = torch.randn(2, 8, 128, device="cuda").bfloat16()
kc = torch.randn(2, 2, 256, 128, device="cuda").bfloat16()
sl = torch.tensor([100, 256], dtype=torch.int32, device="cuda")
ea.decode(qd, kc, kc, sl, chunk=64)
torch.cuda.synchronize()
print("child done", flush=True)
"""


def test_log_lines_when_enabled():
    env = dict(os.environ, MI355ATTN_LOG="1")
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "child done" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("mi355attn: ")]
    print("\n".join(lines))
    want = ["attn_fwd_kernel<fp16,64,causal> grid=2 block=512 B=1 Hq=2 Hkv=2 Nq=128 Nk=128",
            "attn_bwd_dq_kernel<fp16,64,causal> grid=",
            "attn_decode_split_kernel<bf16,128,padded> grid=",
            "attn_decode_combine_kernel<bf16,128> grid=4 block=256 B=2 Hq=8 chunks=4 chunk=64"]
    for w in want:
        assert any(w in l for l in lines), (w, lines)


def test_silent_by_default(capfd):
    if os.environ.get("MI355ATTN_LOG", "") not in ("", "0"):
        pytest.skip("MI355ATTN_LOG is set for this process")
    q = torch.randn(1, 2, 128, 64, device="cuda").half()
    ea.fwd(q, q, q, causal=True)
    torch.cuda.synchronize()
    assert "mi355attn:" not in capfd.readouterr().err
