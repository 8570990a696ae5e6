"""Host logic of bench.py (no GPU): the one-GPU contract, the kernel-trace
parsing behind `split_vs_read_kernel_trace`, and the trace server's
protocol."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = ('"Kind","Agent_Id","Queue_Id","Stream_Id","Thread_Id","Dispatch_Id","Kernel_Id",'
          '"Kernel_Name","Correlation_Id","Start_Timestamp","End_Timestamp","LDS_Block_Size",'
          '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Workgroup_Size_X",'
          '"Workgroup_Size_Y","Workgroup_Size_Z","Grid_Size_X","Grid_Size_Y","Grid_Size_Z"')


def _row(name, start, end, wg_size, grid):
    return (f'"KERNEL_DISPATCH","Agent 1",1,0,1,1,1,"{name}",1,{start},{end},0,0,8,0,32,'
            f'{wg_size},1,1,{grid},1,1')


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_split_read_times_from_a_trace(tmp_path):
    # split kernel launches of 14 and 16 us; reads of 13 us at 1024
    # work-groups and 12 us at 4096: the better read is taken
    rows = [HEADER,
            _row("void kvfp8::paged_decode_split_kernel<128, 1, 4, 2, 1, 1, true, false, "
                 "false, false>(kvfp8::DecodeParams)", 1000, 15000, 256, 65536),
            _row("void kvfp8::paged_decode_split_kernel<128, 1, 4, 2, 1, 1, true, false, "
                 "false, false>(kvfp8::DecodeParams)", 20000, 36000, 256, 65536),
            _row("void kvfp8::paged_decode_reduce_kernel<128, 32>(kvfp8::DecodeParams)",
                 36000, 40000, 64, 4096),
            _row("kvfp8::(anonymous namespace)::stream_read_kernel(unsigned int __vector(4) "
                 "const*, long, unsigned int*)", 50000, 63000, 256, 262144),
            _row("kvfp8::(anonymous namespace)::stream_read_kernel(unsigned int __vector(4) "
                 "const*, long, unsigned int*)", 70000, 82000, 256, 1048576)]
    f = tmp_path / "tp_kernel_trace.csv"
    f.write_text("\n".join(rows) + "\n")
    r = bench.split_read_times([str(f)])
    assert r == dict(split_us=15.0, read_us=12.0, ratio=1.25, split_launches=2)


def test_split_read_times_needs_both_kernels(tmp_path):
    f = tmp_path / "tp_kernel_trace.csv"
    f.write_text(HEADER + "\n" + _row("kvfp8::paged_decode_split_kernel<128>(x)", 0, 1000,
                                      256, 65536) + "\n")
    assert bench.split_read_times([str(f)]) is None
    assert bench.split_read_times([]) is None


def test_kernel_trace_ratios_without_a_server():
    assert bench.kernel_trace_ratios(None) is None


def test_trace_server_answers_every_request():
    # one reply line per request line, malformed requests included; without
    # a GPU (or a profiler) the trace point itself has no result
    srv = bench.start_trace_server()
    assert srv is not None
    try:
        out = bench.kernel_trace_ratios(srv, points=[("bad", None), ("tiny", ["--context", "16"])],
                                        timeout=170)
        assert set(out) == {"bad", "tiny"}
        assert out["bad"] is None
        t = out["tiny"]
        assert t is None or set(t) == {"split_us", "read_us", "ratio", "split_launches"}
    finally:
        bench.stop_trace_server(srv)
    assert srv.poll() is not None
