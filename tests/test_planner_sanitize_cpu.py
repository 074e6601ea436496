"""The host side of the library (argument checks, jagged tile scheduler, workspace layout, C ABI)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven through host-only
plans of every workload and mode, plus the error paths. No kernel code is built: the launchers are
stubs that host-only plans never call. Runs on the CPU."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import jfa_inputs as ji

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GPP = shutil.which("g++")
HIP_INC = "/opt/rocm/include"

STUBS = r"""
#include "jfa_internal.h"
namespace jfa {
hipError_t launch_forward(const FwdArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_forward_combine(const FwdArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dkdv(const BwdArgs&, const Modes&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dq(const BwdArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_reduce_dq(const BwdArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_reduce_dq_wide(const BwdArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_fused(const BwdArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_reduce_dkdv(const BwdArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dbias_clear(const BwdArgs&, const Modes&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dbias_finish(const BwdArgs&, const Modes&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mx_quantize(const MxArgs&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_forward_mx(const MxArgs&, const Modes&, int, hipStream_t) { return hipErrorNotSupported; }
int occupancy_forward(const Modes&) { return 1; }
int occupancy_dq(const Modes&) { return 1; }
int occupancy_dkdv(const Modes&) { return 1; }
}
"""

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "jfa.h"
// stdin: cases of "B H D mask act bias flags slots window block", then B+1 q offsets, B+1 kv offsets
int main() {
  int B, H, D, mask, act, bias, slots, window, block, n = 0;
  unsigned flags;
  while (std::scanf("%d %d %d %d %d %d %u %d %d %d", &B, &H, &D, &mask, &act, &bias, &flags, &slots, &window, &block) == 10) {
    std::vector<int32_t> qo(B + 1), ko(B + 1);
    for (auto& x : qo) if (std::scanf("%d", &x) != 1) return 2;
    for (auto& x : ko) if (std::scanf("%d", &x) != 1) return 2;
    jfa_problem p{};
    p.num_seqs = B; p.num_heads = H; p.head_dim = D; p.q_offsets_host = qo.data(); p.kv_offsets_host = ko.data();
    p.mask = mask; p.act = act; p.bias = bias; p.num_slots = slots; p.flags = flags | JFA_PLAN_HOST_ONLY;
    p.window = window; p.block = block;
    jfa_plan_t plan = nullptr;
    const jfa_status st = jfa_plan(&p, nullptr, &plan);
    std::printf("%d", (int)st);
    if (st == JFA_OK) {
      size_t f = 0, b = 0, total = 0;
      jfa_workspace_bytes(plan, &f, &b);
      for (int w = 0; w < 9; ++w) {
        size_t cnt = 0;
        jfa_plan_schedule(plan, w, nullptr, 0, &cnt);
        std::vector<int32_t> buf(cnt * 6 + 1);
        jfa_plan_schedule(plan, w, buf.data(), cnt, &cnt);
        for (size_t i = 0; i < cnt * ((w & 1) && w < 6 ? 5 : 6); ++i) total += (size_t)buf[i] * (i % 7 + 1);
      }
      int32_t info[9];
      jfa_plan_info(plan, info, 9);
      std::printf(" %zu %zu %zu", f, b, total);
      if (jfa_forward(plan, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != JFA_ERR_HOST_ONLY) return 3;
      jfa_plan_destroy(plan);
    } else {
      std::printf(" %s", jfa_last_error());
    }
    std::printf("\n");
    ++n;
  }
  return n > 0 ? 0 : 1;
}
"""


def _case(lq, lkv, H, D, mask=0, act=0, bias=0, flags=0, slots=0, window=0, block=0):
    qo, ko = ji.offsets(lq), ji.offsets(lkv)
    return (f"{len(lq)} {H} {D} {mask} {act} {bias} {flags} {slots} {window} {block}\n"
            + " ".join(map(str, qo)) + "\n" + " ".join(map(str, ko)) + "\n")


@pytest.mark.skipif(GPP is None or not os.path.exists(os.path.join(HIP_INC, "hip", "hip_runtime.h")),
                    reason="g++ or the HIP headers not available")
def test_planner_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    (tmp_path / "stubs.cpp").write_text(STUBS)
    (tmp_path / "driver.cpp").write_text(DRIVER)
    exe = tmp_path / "planner_asan"
    cmd = [GPP, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INC, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "jagged_sequence_amd", "csrc"),
           os.path.join(ROOT, "jagged_sequence_amd", "csrc", "jfa.cpp"), str(tmp_path / "stubs.cpp"),
           str(tmp_path / "driver.cpp"), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    cases = []
    for name, w in ji.WORKLOADS.items():
        lq, lkv = ji.lengths(w)
        mask = 1 if w.mask == "causal" else 0
        act = ji.ACTS.index(w.act)
        bias = ji.BIASES.index(w.bias)
        flags = (4 if w.shared_q else 0) | (8 if w.mxfp8 else 0)
        for slots in (0, 37):
            cases.append(_case(lq, lkv, w.H, w.D, mask, act, bias, flags, slots, w.window, w.block))
    cases += [
        _case([0, 5, 0], [0, 5, 0], 2, 64, mask=1),                       # empty sequences
        _case([300, 1, 700], [300, 1, 700], 3, 128, mask=1, window=50, block=128, slots=8),
        _case([40, 40], [3, 900], 2, 128, flags=4 | 2),                  # shared queries, no split
        _case([3, 4], [3, 5], 2, 64, mask=1),                            # causal with Lq < Lkv: refused
        _case([3, 4], [3, 4], 2, 96),                                    # bad head dim: refused
        _case([130944], [130944], 64, 128, flags=2),                     # the 32-bit slice limit exactly
        _case([130945], [130945], 64, 128),                              # one row beyond it: refused
    ]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([str(exe)], input="".join(cases), capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.returncode, run.stderr[-4000:])
    lines = run.stdout.strip().split("\n")
    assert len(lines) == len(cases)
    codes = [int(l.split()[0]) for l in lines]
    assert codes[:-4] == [0] * (len(cases) - 4) and codes[-4] == 3 and codes[-3] == 3 and codes[-2] == 0 \
        and codes[-1] == 3, codes
    assert "ERROR: AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr
