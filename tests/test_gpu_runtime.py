"""The HIP library and torch share one HIP runtime in the process, whatever the import
order of the caller (a second runtime would own neither torch's streams nor its memory)."""
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu


def test_library_first_import_order_launches():
    code = (
        "import int4_quantized_kv_amd as kvq\n"
        "import torch\n"
        "x = torch.zeros((1, 1, 8, 128), dtype=torch.float16, device='cuda')\n"
        "d = kvq.make_desc('int4', 1, 1, 128, 8)\n"
        "c = kvq.DeviceCache(d, 'cuda')\n"
        "kvq.kvq_quantize_prefill(d, c.c, x, x, 0, 8)\n"
        "torch.cuda.synchronize()\n"
        "assert float(c.k_scales.sum()) == 16.0\n"   # all-zero groups -> scale 1
        "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
