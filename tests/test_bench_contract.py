"""bench.py's contract checks that need no GPU: the one-GPU refusal and the
algorithmic byte count of the headline workload."""
import json
import os
import subprocess
import sys

import bench
from mxfp4_mixture_experts_amd import synthetic as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def test_headline_algorithmic_bytes():
    """gpt-oss-20b gate_up decode, one token, 4 experts: each touched weight row is
    90 blocks x 16 code bytes + 90 scale bytes + a 2-byte bias (the tensor table's
    layout); x is 2880 bf16; out is 4 x 5760 fp32; the grouping reads E + 1
    offsets and the 4 routed rows."""
    p = S.make_config(1)
    acc = bench.algorithmic(p, 4)
    weights = 4 * 5760 * (90 * 16 + 90 + 2)
    assert acc["weight_bytes"] == weights
    assert acc["proj"] == weights + 2880 * 2 + 4 * 5760 * 4 + 33 * 4 + 4 * 4
    assert acc["flops"] == 2.0 * 4 * 5760 * 2880



def test_published_context_is_quoted_not_compared():
    """The pages' only measured numbers (whole-model decode on an H100) ride
    along in the line as context; no ratio is formed with them."""
    pc = bench.PUBLISHED_CONTEXT
    assert pc["gpt2_124m_decode_tok_s"]["transformers_eager"] == 175.29
    assert pc["gpt2_124m_decode_tok_s"]["transformers_torch_compile"] == 419.13
    assert pc["gpt2_124m_decode_tok_s"]["vllm"] == 696.25
    assert "H100" in pc["note"]
