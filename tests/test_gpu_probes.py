"""Hardware facts the kernels rely on, checked on the device.

- The lane layout of v_mfma_f32_32x32x2_f32 (and 16x16x4) that the MFMA
  kernel's fragment loads and epilogue assume: lane l supplies A(l%32, l/32)
  and B(l/32, l%32); accumulator register i of lane l holds
  D(8*(i/4) + 4*(l/32) + i%4, l%32).
- The LDS bank behaviour the padding and swizzle choices assume: a
  conflict-free access pattern is served at the minimum cost for its width,
  and lanes that share banks cost proportionally more.
"""
import os
import re
import subprocess

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "bin")


def _run(args, timeout=60):
    exe = os.path.join(BIN, args[0])
    if not os.path.exists(exe):
        pytest.fail(f"{exe} is not built (run __graft_entry__.build())")
    proc = subprocess.run([exe, *args[1:]], capture_output=True, text=True, timeout=timeout)
    assert proc.returncode == 0, proc.stderr
    return proc.stdout


def _check_layout(out, nreg, mn, kk, a_map, b_map, c_map):
    bad = 0
    for blk in range(128):
        L, onehot_a = blk & 63, blk < 64
        Am = np.zeros((mn, kk))
        Bm = np.zeros((kk, mn))
        for l in range(64):
            Am[a_map(l)] = (1.0 if l == L else 0.0) if onehot_a else l + 1.0
            Bm[b_map(l)] = l + 1.0 if onehot_a else (1.0 if l == L else 0.0)
        D = Am @ Bm
        for l in range(64):
            for r in range(nreg):
                bad += D[c_map(l, r)] != out[blk, l, r]
    return bad


def test_mfma_lane_layout(tmp_path):
    f = tmp_path / "layout.bin"
    _run(["mfma_layout_probe", str(f)])
    data = np.fromfile(f, dtype=np.float32)
    o32 = data[: 128 * 64 * 16].reshape(128, 64, 16)
    o16 = data[128 * 64 * 16:].reshape(128, 64, 4)
    assert _check_layout(o32, 16, 32, 2, lambda l: (l % 32, l // 32), lambda l: (l // 32, l % 32),
                         lambda l, r: (8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32)) == 0
    assert _check_layout(o16, 4, 16, 4, lambda l: (l % 16, l // 16), lambda l: (l // 16, l % 16),
                         lambda l, r: (4 * (l // 16) + r, l % 16)) == 0


def test_lds_bank_behaviour():
    out = _run(["lds_bank_probe"], timeout=120)
    cyc = {(int(w), int(s)): float(c) for w, s, c in re.findall(r"width=(\d+) stride=(\d+) ms=\S+ cycles=(\S+)", out)}
    print(out)
    # 128-bit reads: 16 lanes x 16 bytes per cycle from 64 banks; 16-byte lane stride is
    # conflict-free, 256-byte stride puts all 16 lanes of a quarter-wave on the same 4 banks.
    assert cyc[(4, 16)] > 8 * cyc[(4, 1)]
    # 32-bit reads: lane strides coprime with the bank count are conflict-free; a 32-word
    # stride puts every lane of a half-wavefront on one bank.
    assert cyc[(1, 32)] > 8 * cyc[(1, 1)]
    assert cyc[(1, 33)] < 1.5 * cyc[(1, 1)]
    assert cyc[(1, 17)] < 1.5 * cyc[(1, 1)]
