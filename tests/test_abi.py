"""The C ABI loads and exports what include/grz.h declares; host-only entry
points (index helpers, argument checks) behave as documented.  No GPU work."""

import ctypes
import os
import re

import pytest

import gradient_reduce_zero_amd as grz
from gradient_reduce_zero_amd import _native as N
from oracle.reduce import chunk_owner, owned_chunk
from oracle.ring import chunk_bounds

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "grz.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z][a-z0-9_]*)\s*\(", text)) -
                  {"defined", "if", "sizeof"})


def test_library_exports_every_declared_symbol():
    lib = grz.lib()
    names = declared_functions()
    assert "dp_reduce_scatter_mean" in names and "zero1_all_gather" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(N.SIGNATURES), "binding signatures out of step with the header"
    assert lib.grz_version() == 103


def test_package_exports_every_flag_and_type_constant():
    for name in dir(N):
        if name.startswith("GRZ_") and not name.startswith("GRZ_E") and name != "GRZ_OK":
            assert getattr(grz, name) == getattr(N, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(r"#define GRZ_MAX_RANKS (\d+)", text).group(1) == str(N.GRZ_MAX_RANKS)
    assert re.search(r"#define GRZ_PIECE (\d+)", text).group(1) == str(N.GRZ_PIECE)
    for name in ("GRZ_SUM", "GRZ_UNEVEN", "GRZ_IN_COMPACT", "GRZ_BF16_WIRE", "GRZ_IN_RANGE",
                 "GRZ_ARGS_DEVICE", "GRZ_OUT_GLOBAL", "GRZ_IN_TILED", "GRZ_MEAN_BF16",
                 "GRZ_COOPERATIVE",
                 "GRZ_EINDIVISIBLE",
                 "GRZ_BF16"):
        assert re.search(rf"{name} = (\d+)", text).group(1) == str(getattr(N, name))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
def test_ownership_helpers_match_oracle(n):
    for r in range(n):
        assert grz.dp_ring_owned_chunk(r, n) == owned_chunk(r, n)
        assert grz.dp_ring_chunk_owner(r, n) == chunk_owner(r, n)
    assert grz.dp_ring_owned_chunk(n, n) == -1
    assert grz.dp_ring_chunk_owner(-1, n) == -1


@pytest.mark.parametrize("length,n", [(64, 3), (0, 4), (7, 8), (4096, 2), (10 ** 12 + 5, 7)])
def test_chunk_range_matches_array_split(length, n):
    for c, (lo, hi) in enumerate(chunk_bounds(length, n)):
        assert grz.dp_chunk_range(length, n, c) == (lo, hi - lo)


def test_piece_numbering():
    buckets = [(10000, 9000), (0, 10000)]
    # bucket 0: chunks of 4500 -> 2 pieces each; bucket 1: 5000 -> 2 each.
    assert grz.dp_piece_count(buckets, 2) == 8
    assert grz.dp_piece_offset(buckets, 2, 0, 1) == 2
    assert grz.dp_piece_offset(buckets, 2, 1, 0) == 4
    assert grz.dp_shard_numel(buckets, 2, 1) == 9500
    # uneven chunks (array_split rule): 64 over 3 -> 22, 21, 21, one piece each
    assert grz.dp_piece_count([(0, 64)], 3) == 3
    assert grz.dp_piece_count([(0, 0)], 4) == 0
    assert grz.dp_grad_sqnorm_workspace(0) == 0
    assert grz.dp_grad_sqnorm_workspace(4096) == 0
    assert grz.dp_grad_sqnorm_workspace(4097) == 16
    assert grz.dp_grad_sqnorm_workspace(4096 * 4096 + 1) == 8 * (4097 + 2)


def _rs(lib, ptrs, n, dtype, buckets, chunk, flags, out):
    arr = (N.Bucket * max(len(buckets), 1))(*buckets)
    pp = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
    return lib.dp_reduce_scatter_mean(pp, n, dtype, arr, len(buckets), chunk, flags, out, None,
                                      None)


def test_argument_errors_return_before_any_launch():
    lib = grz.lib()
    fake = [0x10000, 0x20000]  # never dereferenced: every call below fails validation
    out = ctypes.c_void_p(0x30000)
    assert _rs(lib, fake, 0, N.GRZ_F32, [(0, 64)], 0, 0, out) == N.GRZ_EINVAL
    assert _rs(lib, fake, 2, 7, [(0, 64)], 0, 0, out) == N.GRZ_EINVAL
    assert _rs(lib, fake, 2, N.GRZ_F32, [(0, 63)], 1, 0, out) == N.GRZ_EINDIVISIBLE
    assert _rs(lib, fake, 2, N.GRZ_F32, [(0, 64)], 2, 0, out) == N.GRZ_EINVAL
    assert _rs(lib, fake, 2, N.GRZ_F32, [(0, 64)], -1, N.GRZ_IN_COMPACT, out) == N.GRZ_EINVAL
    assert _rs(lib, fake, 2, N.GRZ_F32, [(-4, 64)], 0, 0, out) == N.GRZ_ERANGE
    assert _rs(lib, fake, 2, N.GRZ_F32, [(0, 64)], 0, 1 << 9, out) == N.GRZ_EINVAL
    assert _rs(lib, fake, 2, N.GRZ_F32, [(0, 64)], 0, N.GRZ_BF16_WIRE, out) == N.GRZ_EINVAL
    both = N.GRZ_IN_RANGE | N.GRZ_IN_COMPACT
    assert _rs(lib, fake, 2, N.GRZ_F32, [(0, 64)], 0, both, out) == N.GRZ_EINVAL
    assert _rs(lib, [0x10001, 0x20000], 2, N.GRZ_F32, [(0, 64)], 0, 0, out) == N.GRZ_EALIGN
    assert _rs(lib, [0x10000, 0], 2, N.GRZ_F32, [(0, 64)], 0, 0, out) == N.GRZ_EINVAL
    assert _rs(lib, fake, 2, N.GRZ_F32, [(0, 64)], 0, 0, None) == N.GRZ_EINVAL
    assert lib.dp_grad_sqnorm(None, 5, 1.0, None, None, None, None) == N.GRZ_EINVAL
    assert lib.dp_grad_sqnorm(ctypes.c_void_p(0x10000), 5000, 1.0, None,
                              ctypes.c_void_p(0x20000), None, None) == N.GRZ_EINVAL
    assert lib.grz_set_max_blocks(0) == N.GRZ_EINVAL
    for code in range(6):
        assert lib.grz_strerror(code)
    assert b"divisible" in lib.grz_strerror(N.GRZ_EINDIVISIBLE)


def test_all_gather_and_out_global_refusals_before_any_launch():
    # dp_all_gather: a dtype outside bf16/fp32/fp64, an unknown flag, a null
    # shard table and a pointer off its element's alignment fail on the host;
    # the optimizer refuses the reduce-only GRZ_OUT_GLOBAL.
    lib = grz.lib()
    b = (N.Bucket * 1)((0, 64))
    shards = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    reps = (ctypes.c_void_p * 1)(0x30000)
    assert lib.dp_all_gather(shards, 2, 7, b, 1, 0, reps, 1, None) == N.GRZ_EINVAL
    assert lib.dp_all_gather(shards, 2, N.GRZ_F32, b, 1, N.GRZ_SUM, reps, 1, None) == N.GRZ_EINVAL
    assert lib.dp_all_gather(None, 2, N.GRZ_F32, b, 1, 0, reps, 1, None) == N.GRZ_EINVAL
    assert lib.dp_all_gather(shards, 17, N.GRZ_F32, b, 1, 0, reps, 1, None) == N.GRZ_EINVAL
    odd = (ctypes.c_void_p * 1)(0x30002)  # 2-byte aligned: fine for bf16, not for fp32
    assert lib.dp_all_gather(shards, 2, N.GRZ_F32, b, 1, 0, odd, 1, None) == N.GRZ_EALIGN
    assert lib.dp_all_gather(shards, 2, N.GRZ_F64, b, 1, 0, (ctypes.c_void_p * 1)(0x30004), 1,
                             None) == N.GRZ_EALIGN
    assert lib.dp_all_gather(shards, 2, N.GRZ_F32, (N.Bucket * 1)((0, 63)), 1, 0, reps, 1,
                             None) == N.GRZ_EINDIVISIBLE
    args = N.AdamWArgs(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)
    assert lib.zero1_adamw_gather(16, 16, 16, 16, b, 1, 2, 0, N.GRZ_OUT_GLOBAL, 16,
                                  ctypes.byref(args), reps, 1, None) == N.GRZ_EINVAL
    assert lib.zero1_fused_step((ctypes.c_void_p * 2)(16, 16), 2, N.GRZ_BF16, b, 1, 0,
                                N.GRZ_OUT_GLOBAL, 16, 16, 16, ctypes.byref(args), 1.0, reps, 1,
                                16, 16, None, None, None, None) == N.GRZ_EINVAL


def test_tiled_receive_buffer_size_and_refusals():
    # GRZ_IN_TILED: one slot of N * GRZ_PIECE elements per piece of the chunk
    # (array_split chunks, the last piece of each bucket's chunk short); only
    # with GRZ_IN_COMPACT, rank pointers exactly one piece apart; refused by
    # the optimizer and the one-launch step.  No call below reaches a launch.
    T = N.GRZ_PIECE
    for buckets, n in (([(10000, 9000), (0, 10000)], 2), ([(0, 64)], 3), ([(0, 0)], 4),
                       ([(5, 3 * T + 1), (0, 5)], 3), ([(0, 16 * 7 * T)], 16)):
        uneven = N.GRZ_UNEVEN if any(length % n for _, length in buckets) else 0
        for c in range(n):
            pieces = sum(-(-(hi - lo) // T) for _, length in buckets
                         for lo, hi in [chunk_bounds(length, n)[c]])
            assert grz.dp_tiled_numel(buckets, n, c, uneven) == pieces * n * T
    lib = grz.lib()
    arr = (N.Bucket * 1)((0, 64))
    assert lib.dp_tiled_numel(arr, 1, 2, -1, 0) == -N.GRZ_EINVAL
    assert lib.dp_tiled_numel(arr, 1, 3, 0, 0) == -N.GRZ_EINDIVISIBLE
    out = ctypes.c_void_p(0x30000)
    tiled = N.GRZ_IN_TILED | N.GRZ_IN_COMPACT
    apart = [0x100000, 0x100000 + 4 * T]  # fp32: one piece apart
    assert _rs(lib, apart, 2, N.GRZ_F32, [(0, 64)], 0, N.GRZ_IN_TILED, out) == N.GRZ_EINVAL
    assert _rs(lib, [0x100000, 0x100000 + 2 * T], 2, N.GRZ_F32, [(0, 64)], 0, tiled,
               out) == N.GRZ_EINVAL
    assert _rs(lib, [0x100000, 0x200000], 2, N.GRZ_BF16, [(0, 64)], 0, tiled,
               out) == N.GRZ_EINVAL
    args = N.AdamWArgs(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)
    reps = (ctypes.c_void_p * 1)(0x30000)
    assert lib.zero1_adamw_gather(16, 16, 16, 16, arr, 1, 2, 0, N.GRZ_IN_TILED, 16,
                                  ctypes.byref(args), reps, 1, None) == N.GRZ_EINVAL
    assert lib.zero1_fused_step((ctypes.c_void_p * 2)(16, 16), 2, N.GRZ_BF16, arr, 1, 0, tiled,
                                16, 16, 16, ctypes.byref(args), 1.0, reps, 1, 16, 16, None,
                                None, None, None) == N.GRZ_EINVAL


def test_bf16_mean_refusals():
    # GRZ_MEAN_BF16: the rounding of an fp32 mean, so refused for fp64
    # gradients; a bf16 mean needs 2-byte alignment only; refused by the
    # all-gathers and the one-launch step.  No call below reaches a launch.
    lib = grz.lib()
    arr = (N.Bucket * 1)((0, 64))
    out = ctypes.c_void_p(0x30000)
    f = N.GRZ_MEAN_BF16
    assert _rs(lib, [0x100000, 0x200000], 2, N.GRZ_F64, [(0, 64)], 0, f, out) == N.GRZ_EINVAL
    assert _rs(lib, [0x100000, 0x200000], 2, N.GRZ_BF16, [(0, 64)], 0, f,
               ctypes.c_void_p(0x30001)) == N.GRZ_EALIGN
    assert _rs(lib, [0x100000, 0x200000], 2, N.GRZ_BF16, [(0, 64)], 0, 0,
               ctypes.c_void_p(0x30002)) == N.GRZ_EALIGN
    args = N.AdamWArgs(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)
    reps = (ctypes.c_void_p * 1)(0x30000)
    assert lib.zero1_adamw_gather(16, 16, 16, 0x30001, arr, 1, 2, 0, f, 16,
                                  ctypes.byref(args), reps, 1, None) == N.GRZ_EALIGN
    assert lib.zero1_all_gather((ctypes.c_void_p * 2)(16, 16), 2, arr, 1, f, reps, 1,
                                None) == N.GRZ_EINVAL
    assert lib.zero1_fused_step((ctypes.c_void_p * 2)(16, 16), 2, N.GRZ_BF16, arr, 1, 0,
                                f | N.GRZ_IN_COMPACT, 16, 16, 16, ctypes.byref(args), 1.0, reps,
                                1, 16, 16, None, None, None, None) == N.GRZ_EINVAL


C_CALLER = r"""
#include <stdio.h>
#include "grz.h"
int main(void) {
  grz_bucket b[1] = {{0, 64}};
  int64_t off = -1, n = -1;
  dp_chunk_range(10, 3, 1, &off, &n);
  printf("%d %d %d %lld %lld %lld\n", grz_version(), dp_ring_owned_chunk(0, 8),
         dp_ring_chunk_owner(0, 8), (long long)off, (long long)n,
         (long long)dp_piece_count(b, 1, 2, 0));
  return 0;
}
"""


def test_header_is_c_and_a_c_program_links_the_library(tmp_path):
    # The boundary is a C ABI: grz.h compiles as C11 with warnings as errors,
    # and a C program linked against libgrz.so calls its host-only helpers
    # (no device work): ring ownership (rank r owns chunk r + 1 mod N), an
    # array_split chunk (10 over 3: chunk 1 is [4, 7)), one piece per chunk.
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src, exe = tmp_path / "caller.c", tmp_path / "caller"
    src.write_text(C_CALLER)
    libdir = os.path.dirname(N.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.dirname(HEADER)}", "-I/opt/rocm/include", str(src),
           f"-L{libdir}", "-lgrz", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == [str(grz.lib().grz_version()), "1", "7", "4", "3", "2"]


def test_reduce_refuses_the_flags_of_other_entry_points():
    # The reduce (and its _range and _weighted forms) takes neither
    # GRZ_ARGS_DEVICE nor GRZ_COOPERATIVE; refused before any launch.
    lib = grz.lib()
    arr = (N.Bucket * 1)((0, 64))
    pp = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    out = ctypes.c_void_p(0x30000)
    counts = (ctypes.c_int64 * 2)(3, 5)
    for f in (N.GRZ_ARGS_DEVICE, N.GRZ_COOPERATIVE, 1 << 12):
        assert _rs(lib, [0x100000, 0x200000], 2, N.GRZ_BF16, [(0, 64)], 0, f, out) == \
            N.GRZ_EINVAL
        assert lib.dp_reduce_scatter_mean_range(pp, 2, N.GRZ_BF16, arr, 1, 0, 1, 0, f, out,
                                                None, None) == N.GRZ_EINVAL
        assert lib.dp_reduce_scatter_weighted(pp, counts, 2, N.GRZ_BF16, arr, 1, 0, 1, 0, f,
                                              out, None, None) == N.GRZ_EINVAL


def test_product_path_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        grz.dp_reduce_scatter_mean([torch.zeros(64), torch.zeros(64)], [(0, 64)], 0,
                                   torch.zeros(32))


def test_norm_and_fused_workspace_sizes():
    assert grz.dp_grad_sqnorm_of_workspace(0) == 0
    assert grz.dp_grad_sqnorm_of_workspace(1) == 8
    assert grz.dp_grad_sqnorm_of_workspace(4096 * 4097) == 4097 * 8 + 2 * 8
    ctl = 256  # control words; then one published slot per piece, per level sum, the norm
    assert grz.zero1_fused_workspace(0) == ctl + 8
    assert grz.zero1_fused_workspace(4096) == ctl + (4096 + 1) * 8
    assert grz.zero1_fused_workspace(4097) == ctl + (4097 + 2 + 1) * 8
    assert grz.zero1_fused_workspace(4096 * 4096) == ctl + (4096 * 4096 + 4096 + 1) * 8


def test_fused_step_refusals_before_any_launch():
    # Checked on the host before anything touches a device: unknown flags, the
    # sum and bf16-wire modes, a bad N, a null state pointer.
    lib = grz.lib()
    b = (N.Bucket * 1)((0, 64))
    ptrs = (ctypes.c_void_p * 2)(16, 16)
    reps = (ctypes.c_void_p * 1)(16)
    args = N.AdamWArgs(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)

    def call(nranks=2, flags=0, master=16):
        return lib.zero1_fused_step(ptrs, nranks, N.GRZ_BF16, b, 1, 0, flags, master, 16, 16,
                                    ctypes.byref(args), 1.0, reps, 1, 16, 16, None, None,
                                    None, None)

    for flags in (N.GRZ_SUM, N.GRZ_BF16_WIRE, N.GRZ_IN_RANGE, 1 << 10):
        assert call(flags=flags) == N.GRZ_EINVAL
    assert call(nranks=17) == N.GRZ_EINVAL
    assert call(master=None) == N.GRZ_EINVAL

    # The form that takes its step scalars from a table: GRZ_ARGS_DEVICE is
    # implied, and the table, its size and the counter are checked.
    def call_args(flags=0, table=0x20000, count=4, counter=0x30000, current=0x40000):
        return lib.zero1_fused_step_args(ptrs, 2, N.GRZ_BF16, b, 1, 0, flags, 16, 16, 16, table,
                                         count, counter, current, 1.0, reps, 1, 16, 16, None,
                                         None, None, None)

    assert call_args(flags=N.GRZ_ARGS_DEVICE) == N.GRZ_EINVAL
    assert call_args(flags=N.GRZ_SUM) == N.GRZ_EINVAL
    assert call_args(table=None) == N.GRZ_EINVAL
    assert call_args(count=0) == N.GRZ_EINVAL
    assert call_args(counter=None) == N.GRZ_EINVAL
    assert call_args(counter=0x30004) == N.GRZ_EALIGN
    assert lib.zero1_fused_capacity(0, N.GRZ_BF16) == -N.GRZ_EINVAL
    assert lib.zero1_fused_capacity(2, N.GRZ_F64) == -N.GRZ_EINVAL


def test_missing_library_fails_loudly(tmp_path):
    # No fallback of any kind: without libgrz.so every entry point raises.
    import subprocess
    import sys
    code = (
        "import gradient_reduce_zero_amd._native as N\n"
        f"N.LIB_PATH = {str(tmp_path / 'libgrz.so')!r}\n"
        "import gradient_reduce_zero_amd as grz\n"
        "try:\n"
        "    grz.dp_piece_count([(0, 64)], 2)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=root, timeout=120)
    assert res.returncode == 0, res.stderr
    assert "raised:" in res.stdout and "no fallback" in res.stdout


# Random plans: the library's host-side plan arithmetic against the oracle's
# chunking (chunk_bounds, shard_segments) and the piece numbering of the norm
# (pieces of GRZ_PIECE elements inside each chunk, numbered bucket by bucket,
# chunk 0..N-1, piece by piece).
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402


@st.composite
def _plans(draw):
    n = draw(st.integers(1, 16))
    even = draw(st.booleans())
    lengths = draw(st.lists(st.integers(0, 3 * 4096 + 50), min_size=1, max_size=6))
    if even:
        lengths = [l - l % n for l in lengths]
    order = draw(st.permutations(range(len(lengths))))
    offs, pos = [0] * len(lengths), 0
    for i in order:  # the arena layout differs from the processing order
        offs[i] = pos
        pos += lengths[i]
    return n, even, list(zip(offs, lengths))


@settings(max_examples=300, deadline=None)
@given(_plans())
def test_plan_helpers_match_the_oracle_on_random_plans(plan):
    from oracle.reduce import shard_segments

    n, even, buckets = plan
    flags = 0 if even else N.GRZ_UNEVEN
    piece = N.GRZ_PIECE
    total = 0
    for b, (_, length) in enumerate(buckets):
        bounds = chunk_bounds(length, n)
        for c, (lo, hi) in enumerate(bounds):
            assert grz.dp_chunk_range(length, n, c) == (lo, hi - lo)
            assert grz.dp_piece_offset(buckets, n, b, c, flags) == total
            total += -(-(hi - lo) // piece)
    assert grz.dp_piece_count(buckets, n, flags) == total
    for c in range(n):
        segs = shard_segments(buckets, n, c, uneven=not even)
        assert grz.dp_shard_numel(buckets, n, c, flags) == sum(s[1] for s in segs)
    if not even and any(l % n for _, l in buckets):
        with pytest.raises(grz.GrzError):
            grz.dp_shard_numel(buckets, n, 0, 0)
