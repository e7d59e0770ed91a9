#!/usr/bin/env python3
"""Calibration launches for the HBM-traffic counters.

Runs the plain 16-byte copy kernel of libceiling.so over a buffer of known size
(default 1 GiB read + 1 GiB written per launch) a few times. Profiled with
`rocprofv3 --pmc FETCH_SIZE` and then `--pmc WRITE_SIZE`, its per-dispatch
readings divided by the bytes it actually moves give the factors that turn the
same counters on other kernels into bytes. Also prints the copy bandwidth.
"""
import argparse
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--bytes", type=int, default=1 << 30)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "ceiling", "libceiling.so"))
    L.ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                               ctypes.c_void_p]
    L.ceiling_copy.restype = ctypes.c_int
    src = torch.empty(args.bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(args.bytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    for _ in range(args.reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        rc = L.ceiling_copy(dst.data_ptr(), src.data_ptr(), args.bytes, 256 * 16,
                            ctypes.c_void_p(s.cuda_stream))
        b.record(s)
        b.synchronize()
        if rc != 0:
            sys.exit(f"ceiling_copy failed: {rc}")
        ms = a.elapsed_time(b)
        print(f"copy {args.bytes} B: {ms * 1e3:.1f} us, {2 * args.bytes / (ms / 1e3) / 1e9:.1f} GB/s "
              "(read + write)", flush=True)


if __name__ == "__main__":
    main()
