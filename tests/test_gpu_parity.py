"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Tolerances: |gpu - ref| <= 2e-3 * max(1, |ref|) for fp16 outputs and 1e-2 * max(1, |ref|)
for bf16 outputs; the W8A8 int32 accumulator bit-exact.  Small cases span several tiles with
ragged edges; the full-size workloads run in the configuration the benchmark times.  Every
output element is compared, except in the two tests whose outputs pass 2^31 elements, which
compare sampled rows.
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (dev_tensor, ref_antiquant, ref_w8a8, run_antiquant, run_w8a8, sampled_rows,
                      to_f64)

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[gpu-case] {name}", flush=True)
    sys.stdout.flush()


def check_aq(case, rows=None):
    _announce(case.name)
    y = run_antiquant(case)
    got = to_f64(y).reshape(-1, case.n)
    if rows is not None:
        got = got[rows]
    ref = ref_antiquant(case, rows).reshape(got.shape)
    r = oracle.compare(got, ref, case.act)
    assert r["ok"], (case.name, r)
    return r


# (name, act, weight, x1 shape, n, mode, group size, extra kwargs)
AQ_CASES = [
    ("c1_tiny_pertensor", None),
    ("perchannel_bf16_i8_ragged", dict(act="bf16", weight="int8", x1_shape=(600, 288), n=544, mode="channel")),
    ("perchannel_bf16_i8_1xn_nooff", dict(act="bf16", weight="int8", x1_shape=(300, 256), n=256, mode="channel",
                                          channel_2d=True, with_offset=False, with_bias=False, with_x3=False)),
    ("perchannel_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(257, 320), n=288, mode="channel")),
    ("pertensor_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(260, 256), n=320, mode="tensor")),
    ("perchannel_fp16_i4", dict(act="fp16", weight="int4", x1_shape=(130, 384), n=192, mode="channel")),
    ("pergroup128_bf16_i4_3d", dict(act="bf16", weight="int4", x1_shape=(2, 300, 512), n=320, mode="group",
                                    group_size=128, scale_dist=("uniform", 0.01, 0.05),
                                    offset_dist=("uniform", -1, 1), with_bias=False)),
    ("pergroup64_fp16_i8_m33", dict(act="fp16", weight="int8", x1_shape=(33, 576), n=256, mode="group",
                                    group_size=64, offset_dist=("uniform", -4, 4))),
    ("pergroup96_bf16_i8_partial", dict(act="bf16", weight="int8", x1_shape=(280, 320), n=160, mode="group",
                                        group_size=96)),
    ("pergroup32_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(100, 256), n=128, mode="group",
                                group_size=32)),
    ("pergroup224_bf16_i8_gkm1", dict(act="bf16", weight="int8", x1_shape=(70, 256), n=96, mode="group",
                                      group_size=224)),
    ("pergroup64_bf16_i8_k96", dict(act="bf16", weight="int8", x1_shape=(40, 96), n=64, mode="group",
                                    group_size=64)),
    ("perchannel_bf16_i8_longk", dict(act="bf16", weight="int8", x1_shape=(256, 4096), n=256, mode="channel")),
    ("pergroup512_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(64, 2048), n=128, mode="group",
                                 group_size=512)),
    # no offset: the row sums' term is s * (0 - C) * S, non-zero for bf16 images of int4
    # codes (C = 136), so those keep the sums (per-channel in the k loop, per-group in the
    # pass before the product); exact images (C = 0) skip them
    ("nooff_perchannel_bf16_i4_c136", dict(act="bf16", weight="int4", x1_shape=(300, 512), n=256,
                                           mode="channel", with_offset=False)),
    ("nooff_pergroup128_bf16_i4_c136", dict(act="bf16", weight="int4", x1_shape=(300, 1024), n=256,
                                            mode="group", group_size=128, with_offset=False)),
    ("nooff_pergroup64_bf16_i8_exact", dict(act="bf16", weight="int8", x1_shape=(300, 1024), n=256,
                                            mode="group", group_size=64, with_offset=False)),
    ("nooff_pergroup96_fp16_i4_exact_splitk", dict(act="fp16", weight="int4", x1_shape=(100, 2304), n=384,
                                                   mode="group", group_size=96, with_offset=False)),
    # groups of 3008 k: three splits of one group each, the last partial
    ("pergroup3008_fp16_i8_long", dict(act="fp16", weight="int8", x1_shape=(300, 8192), n=256, mode="group",
                                       group_size=3008)),
    # many short groups on wide tiles without a k split (5 x 32 tiles fill the CUs): 64 groups
    # of 32 with bf16 images of int4 codes (C = 136, no offset), 72 groups with an offset
    ("pergroup32_bf16_i4_sg64", dict(act="bf16", weight="int4", x1_shape=(520, 2048), n=8192, mode="group",
                                     group_size=32, with_offset=False, scale_dist=("uniform", 0.01, 0.05))),
    ("pergroup32_fp16_i8_pass72", dict(act="fp16", weight="int8", x1_shape=(520, 2304), n=8192, mode="group",
                                       group_size=32, offset_dist=("uniform", -4, 4))),
    # small-m (split-k) path
    ("smallm_pergroup64_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(32, 1024), n=384, mode="group",
                                       group_size=64, offset_dist=("uniform", -4, 4), with_x3=False)),
    ("smallm_m1_perchannel_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(1, 512), n=256, mode="channel")),
    ("smallm_m3_pergroup128_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(3, 1024), n=256, mode="group",
                                           group_size=128)),
    ("smallm_m17_pertensor_fp16_i4", dict(act="fp16", weight="int4", x1_shape=(17, 320), n=128, mode="tensor")),
    # small m at n >= 8192 with k > 1024 (split k over 128-column slabs): ragged k, a 32-row
    # k tail, every mode, fp8, 3-D x1, n not a multiple of the slab
    ("wide_m32_pergroup64_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(32, 1088), n=8192, mode="group",
                                           group_size=64, offset_dist=("uniform", -4, 4))),
    ("wide_m5_perchannel_bf16_i8_k1056", dict(act="bf16", weight="int8", x1_shape=(5, 1056), n=8192,
                                                mode="channel")),
    ("wide_m1_pertensor_fp16_i8_nooff", dict(act="fp16", weight="int8", x1_shape=(1, 2048), n=8192,
                                               mode="tensor", with_offset=False, with_x3=False)),
    ("wide_m17_perchannel_bf16_f8_n8224", dict(act="bf16", weight="fp8e4m3", x1_shape=(17, 1536), n=8224,
                                                 mode="channel", with_offset=False, with_bias=False)),
    ("wide_3d_pergroup32_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(2, 4, 1152), n=8192, mode="group",
                                          group_size=32)),
    ("wide_m32_pergroup96_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(32, 1056), n=8192, mode="group",
                                           group_size=96, with_bias=False)),
    ("smallm_m5_pergroup96_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(5, 544), n=160, mode="group",
                                          group_size=96)),
    ("smallm_m8_pergroup64_bf16_i8_k96", dict(act="bf16", weight="int8", x1_shape=(8, 96), n=64, mode="group",
                                              group_size=64)),
    ("smallm_3d_perchannel_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(2, 4, 2048), n=640,
                                          mode="channel")),
    # the largest k and n the shape rules allow (k, n <= 65535, multiples of 32 / 64)
    ("maxk_smallm_pergroup32_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(3, 65504), n=64, mode="group",
                                            group_size=32)),
    ("maxk_pergroup128_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(96, 65472), n=128, mode="group",
                                      group_size=128, with_bias=False)),
    ("maxn_perchannel_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(40, 64), n=65504, mode="channel")),
    ("maxn_smallm_pertensor_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(8, 64), n=65504, mode="tensor")),
    # m >= 1024: several row tiles share each weight tile (ragged m and n tiles; k not a
    # multiple of 64; the largest k and n at this m)
    ("largem_perchannel_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(1100, 288), n=544, mode="channel")),
    ("largem_pertensor_fp16_i4", dict(act="fp16", weight="int4", x1_shape=(1030, 256), n=320, mode="tensor")),
    ("largem_perchannel_fp16_i8_3d_nooff", dict(act="fp16", weight="int8", x1_shape=(2, 600, 384), n=256,
                                                mode="channel", channel_2d=True, with_offset=False)),
    ("largem_perchannel_bf16_i4_nox3", dict(act="bf16", weight="int4", x1_shape=(1280, 640), n=192, mode="channel",
                                            with_x3=False, with_bias=False)),
    ("largem_maxk_perchannel_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(1024, 65504), n=64,
                                            mode="channel")),
    ("largem_maxn_pertensor_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(1024, 64), n=65504,
                                           mode="tensor")),
    # 32 < m with few output tiles: k is split so that the workgroups fill the CUs, and a
    # finishing kernel adds the fp32 partials (ragged m and n tiles; k with a 32-row tail;
    # per-group splits on group boundaries, 96-wide groups in units of 192)
    ("midm_m64_perchannel_bf16_i8_splitk", dict(act="bf16", weight="int8", x1_shape=(64, 4096), n=512,
                                                mode="channel")),
    ("midm_m100_pergroup96_fp16_i8_splitk", dict(act="fp16", weight="int8", x1_shape=(100, 2304), n=384,
                                                 mode="group", group_size=96, offset_dist=("uniform", -4, 4))),
    ("midm_m129_perchannel_fp16_i8_splitk_tail", dict(act="fp16", weight="int8", x1_shape=(129, 2080), n=256,
                                                      mode="channel")),
    ("midm_m200_pergroup128_bf16_i4_splitk", dict(act="bf16", weight="int4", x1_shape=(200, 2048), n=320,
                                                  mode="group", group_size=128, with_bias=False)),
    ("midm_m300_pertensor_bf16_i8_splitk", dict(act="bf16", weight="int8", x1_shape=(300, 1024), n=256,
                                                mode="tensor")),
    ("midm_m48_perchannel_bf16_f8_splitk", dict(act="bf16", weight="fp8e4m3", x1_shape=(48, 3072), n=288,
                                                mode="channel", with_offset=False,
                                                scale_dist=("uniform", 2e-4, 1e-3))),
    ("midm_xt_m64_pergroup64_bf16_i8_splitk", dict(act="bf16", weight="int8", x1_shape=(64, 2048), n=256,
                                                   mode="group", group_size=64, x2_transposed=True)),
    ("midm_xt_m96_perchannel_fp16_i4_splitk", dict(act="fp16", weight="int4", x1_shape=(96, 2048), n=384,
                                                   mode="channel", x2_transposed=True)),
    # m <= 64: the 64-row tile (per-group row sums as quarter-wave loads)
    ("midm_m40_pergroup96_bf16_i8_xt_splitk", dict(act="bf16", weight="int8", x1_shape=(40, 2304), n=320,
                                                   mode="group", group_size=96, x2_transposed=True)),
    ("midm_m50_pertensor_fp16_i8_splitk", dict(act="fp16", weight="int8", x1_shape=(50, 1600), n=224,
                                               mode="tensor", with_x3=False)),
    ("midm_m64_pergroup64_fp16_i4_splitk", dict(act="fp16", weight="int4", x1_shape=(2, 32, 2048), n=256,
                                                mode="group", group_size=64, with_bias=False)),
    ("midm_m57_perchannel_bf16_f8_nosplit", dict(act="bf16", weight="fp8e4m3", x1_shape=(57, 256), n=96,
                                                 mode="channel", with_offset=False,
                                                 scale_dist=("uniform", 2e-4, 1e-3))),
    # 64 < m <= 128 whose 128-row tiles would split k into chunks of at most 512: two 64-row
    # tiles (the second ragged), every mode and weight type
    ("midm_m96_pergroup128_bf16_i4_rows64", dict(act="bf16", weight="int4", x1_shape=(96, 2048), n=512,
                                                 mode="group", group_size=128)),
    ("midm_m72_perchannel_bf16_f8_rows64", dict(act="bf16", weight="fp8e4m3", x1_shape=(72, 1024), n=256,
                                                mode="channel", with_offset=False,
                                                scale_dist=("uniform", 2e-4, 1e-3))),
    ("midm_m128_pertensor_fp16_i8_rows64", dict(act="fp16", weight="int8", x1_shape=(2, 64, 4096), n=768,
                                                mode="tensor")),
    ("midm_xt_m120_pergroup64_fp16_i8_rows64", dict(act="fp16", weight="int8", x1_shape=(120, 1536), n=320,
                                                    mode="group", group_size=64, x2_transposed=True)),
    # m > 128 whose 256-row tiles would split k into chunks of at most 512: several 128-row
    # tiles (ragged last row tile), per-tensor / per-channel, every weight type, both x2 layouts
    ("midm_m160_perchannel_bf16_i8_rows128", dict(act="bf16", weight="int8", x1_shape=(160, 2048), n=512,
                                                  mode="channel")),
    ("midm_m256_pertensor_fp16_i4_rows128", dict(act="fp16", weight="int4", x1_shape=(4, 64, 1024), n=768,
                                                 mode="tensor")),
    ("midm_m333_perchannel_bf16_f8_rows128", dict(act="bf16", weight="fp8e4m3", x1_shape=(333, 1536), n=320,
                                                  mode="channel", with_offset=False,
                                                  scale_dist=("uniform", 2e-4, 1e-3))),
    ("midm_xt_m390_perchannel_fp16_i8_rows128", dict(act="fp16", weight="int8", x1_shape=(390, 1024), n=640,
                                                     mode="channel", x2_transposed=True, with_bias=False)),
    ("midm_xt_m201_pertensor_bf16_i4_rows128", dict(act="bf16", weight="int4", x1_shape=(201, 4096), n=256,
                                                    mode="tensor", x2_transposed=True)),
    # x2 stored transposed, (n, k) (int4 packed along k), handed over as its (k, n) transpose
    # view; per-group scale and offset transposed with it
    ("xt_perchannel_bf16_i8_ragged", dict(act="bf16", weight="int8", x1_shape=(600, 288), n=544, mode="channel",
                                          x2_transposed=True)),
    ("xt_pergroup128_fp16_i4_3d", dict(act="fp16", weight="int4", x1_shape=(2, 150, 512), n=320, mode="group",
                                       group_size=128, x2_transposed=True)),
    ("xt_pergroup96_bf16_i8_partial", dict(act="bf16", weight="int8", x1_shape=(280, 320), n=160, mode="group",
                                           group_size=96, x2_transposed=True)),
    ("xt_pertensor_bf16_i4_nooff", dict(act="bf16", weight="int4", x1_shape=(260, 256), n=192, mode="tensor",
                                        with_offset=False, x2_transposed=True)),
    ("xt_perchannel_fp16_f8", dict(act="fp16", weight="fp8e4m3", x1_shape=(257, 320), n=288, mode="channel",
                                   with_offset=False, scale_dist=("uniform", 2e-4, 1e-3), x2_transposed=True)),
    ("xt_largem_perchannel_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(1100, 288), n=544,
                                          mode="channel", x2_transposed=True)),
    ("xt_smallm_pergroup64_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(32, 1024), n=384, mode="group",
                                          group_size=64, offset_dist=("uniform", -4, 4), with_x3=False,
                                          x2_transposed=True)),
    ("xt_smallm_m3_pergroup128_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(3, 1024), n=256, mode="group",
                                              group_size=128, x2_transposed=True)),
    ("xt_smallm_m8_pergroup64_bf16_i8_k96", dict(act="bf16", weight="int8", x1_shape=(8, 96), n=64, mode="group",
                                                 group_size=64, x2_transposed=True)),
    ("xt_smallm_m1_perchannel_bf16_f8", dict(act="bf16", weight="fp8e4m3", x1_shape=(1, 512), n=256,
                                             mode="channel", with_offset=False,
                                             scale_dist=("uniform", 2e-4, 1e-3), x2_transposed=True)),
    ("xt_maxk_smallm_pergroup32_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(3, 65504), n=64,
                                               mode="group", group_size=32, x2_transposed=True)),
    ("xt_maxn_perchannel_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(40, 64), n=65472, mode="channel",
                                        x2_transposed=True)),
    # FLOAT8_E4M3FN weights: per-channel, no offset; codes uniform over the finite patterns
    # (zeros of both signs, subnormals, +-448), scales of the size an fp8 weight needs
    ("perchannel_bf16_f8_ragged", dict(act="bf16", weight="fp8e4m3", x1_shape=(600, 288), n=544, mode="channel",
                                       with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("perchannel_fp16_f8_1xn", dict(act="fp16", weight="fp8e4m3", x1_shape=(257, 320), n=288, mode="channel",
                                    channel_2d=True, with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("perchannel_fp16_f8_3d_nobias", dict(act="fp16", weight="fp8e4m3", x1_shape=(3, 70, 512), n=96,
                                          mode="channel", with_offset=False, with_bias=False,
                                          scale_dist=("uniform", 2e-4, 1e-3))),
    ("perchannel_bf16_f8_longk", dict(act="bf16", weight="fp8e4m3", x1_shape=(256, 4096), n=256, mode="channel",
                                      with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("smallm_m1_perchannel_bf16_f8", dict(act="bf16", weight="fp8e4m3", x1_shape=(1, 512), n=256, mode="channel",
                                          with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("smallm_m32_perchannel_fp16_f8", dict(act="fp16", weight="fp8e4m3", x1_shape=(32, 2048), n=640,
                                           mode="channel", with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("smallm_m7_perchannel_fp16_f8_k96", dict(act="fp16", weight="fp8e4m3", x1_shape=(7, 96), n=64, mode="channel",
                                              with_offset=False, with_x3=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("maxk_perchannel_bf16_f8", dict(act="bf16", weight="fp8e4m3", x1_shape=(96, 65504), n=128, mode="channel",
                                     with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("largem_perchannel_bf16_f8", dict(act="bf16", weight="fp8e4m3", x1_shape=(1500, 512), n=96, mode="channel",
                                       with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("largem_perchannel_fp16_f8_1xn", dict(act="fp16", weight="fp8e4m3", x1_shape=(1060, 320), n=288,
                                           mode="channel", channel_2d=True, with_offset=False,
                                           scale_dist=("uniform", 2e-4, 1e-3))),
    ("maxk_smallm_perchannel_fp16_f8", dict(act="fp16", weight="fp8e4m3", x1_shape=(3, 65504), n=64,
                                            mode="channel", with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
]


@pytest.mark.parametrize("name,spec", AQ_CASES, ids=[c[0] for c in AQ_CASES])
def test_antiquant_parity(name, spec):
    if spec is None:
        case = workloads.make_workload("tiny_pertensor_fp16_int8_16x256x256")
    else:
        case = workloads.make_antiquant(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    check_aq(case)


def test_page_sample_antiquant_all_ones():
    import torch
    import weight_quantized_gemm_amd as W
    _announce("page_sample_antiquant")
    d = "cuda:0"
    h = lambda *s: torch.ones(*s, dtype=torch.float16, device=d)
    y = W.antiquant_matmul(h(32, 64), torch.ones(64, 128, dtype=torch.int8, device=d), h(128),
                           h(128), h(128), h(32, 128))
    assert torch.all(y.float() == 130)


@pytest.mark.parametrize("act", ["fp16", "bf16"])
def test_empty_k(act):
    import torch
    import weight_quantized_gemm_amd as W
    _announce(f"empty_k_{act}")
    case = workloads.make_antiquant(seed=7, act=act, weight="int8", x1_shape=(32, 0), n=128, mode="channel")
    y = run_antiquant(case)
    ref = ref_antiquant(case)
    assert oracle.compare(to_f64(y), ref, act)["ok"]
    case0 = workloads.make_antiquant(seed=8, act=act, weight="int8", x1_shape=(32, 0), n=128, mode="channel",
                                     with_bias=False, with_x3=False)
    assert np.all(to_f64(run_antiquant(case0)) == 0)


@pytest.mark.parametrize("m", [4, 40, 1100])
def test_fp8_nan_code(m):
    """FLOAT8_E4M3FN has one NaN pattern per sign (S.1111.111).  Its decoded value enters the
    formula like any other, so its output column is NaN on every row; the other columns
    match the oracle.  The small-m path (m <= 32) and the tiled path, with one and with
    several row tiles."""
    _announce(f"fp8_nan_code_m{m}")
    case = workloads.make_antiquant(seed=31 + m, act="bf16", weight="fp8e4m3", x1_shape=(m, 256), n=128,
                                    mode="channel", with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))
    case.x2[5, 7] = 0x7F
    case.x2[200, 100] = 0xFF
    got = to_f64(run_antiquant(case)).reshape(m, case.n)
    ref = ref_antiquant(case).reshape(m, case.n)
    nan_cols = [7, 100]
    assert np.isnan(ref[:, nan_cols]).all()
    assert np.isnan(got[:, nan_cols]).all()
    keep = np.setdiff1d(np.arange(case.n), nan_cols)
    r = oracle.compare(got[:, keep], ref[:, keep], case.act)
    assert r["ok"], r


def test_fp8_empty_k():
    _announce("fp8_empty_k")
    case = workloads.make_antiquant(seed=9, act="fp16", weight="fp8e4m3", x1_shape=(32, 0), n=128,
                                    mode="channel", with_offset=False)
    assert oracle.compare(to_f64(run_antiquant(case)), ref_antiquant(case), "fp16")["ok"]


def test_determinism():
    _announce("determinism")
    for name, spec in [("det_group", dict(act="bf16", weight="int4", x1_shape=(300, 512), n=320, mode="group",
                                          group_size=128)),
                       ("det_smallm", dict(act="fp16", weight="int8", x1_shape=(32, 2048), n=256, mode="group",
                                           group_size=64))]:
        case = workloads.make_antiquant(seed=5, name=name, **spec)
        a = run_antiquant(case).cpu()
        b = run_antiquant(case).cpu()
        assert bytes(a.view(-1).view(__import__("torch").int16).numpy()) == \
            bytes(b.view(-1).view(__import__("torch").int16).numpy())


def test_smallm_workspace_reuse():
    """One workspace (the small-m split-k partials) serves consecutive calls on different
    inputs and parameter modes; every call is checked against the oracle."""
    import torch
    import weight_quantized_gemm_amd as W
    _announce("smallm_workspace_reuse")
    ws = None
    for i, (mode, g) in enumerate([("group", 64), ("group", 64), ("channel", 0), ("group", 96)]):
        case = workloads.make_antiquant(seed=700 + i, name=f"reuse{i}", act="fp16", weight="int8",
                                        x1_shape=(24, 2304), n=384, mode=mode, group_size=g)
        act = case.act
        call_args = (dev_tensor(case.x1, act), dev_tensor(case.x2, "raw"), dev_tensor(case.scale, act),
                     dev_tensor(case.offset, act), dev_tensor(case.bias, act), dev_tensor(case.x3, act),
                     case.group_size)
        call = W.AntiquantMatmul(*call_args, workspace=ws)
        assert call.workspace_size > 0  # the split-k path
        ws = call.workspace
        y = call()
        torch.cuda.synchronize()
        r = oracle.compare(to_f64(y).reshape(case.out_shape), ref_antiquant(case), act)
        assert r["ok"], (i, r)


def _antiquant_tensors(case):
    act = case.act
    return dict(x1=dev_tensor(case.x1, act), x2=dev_tensor(case.x2, "raw"), scale=dev_tensor(case.scale, act),
                offset=dev_tensor(case.offset, act), bias=dev_tensor(case.bias, act), x3=dev_tensor(case.x3, act))


@pytest.mark.parametrize("name,spec", [
    ("graph_smallm_pergroup64_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(16, 2048), n=384, mode="group",
                                             group_size=64)),
    ("graph_largem_pergroup128_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(300, 512), n=256,
                                              mode="group", group_size=128)),
    ("graph_largem_perchannel_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(260, 256), n=320,
                                             mode="channel")),
    # split k: the finishing kernel is captured with the main kernel
    ("graph_splitk_perchannel_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(96, 2048), n=256,
                                             mode="channel")),
    ("graph_splitk_pergroup128_fp16_i4", dict(act="fp16", weight="int4", x1_shape=(64, 2048), n=256,
                                              mode="group", group_size=128)),
    # m > 128 on 128-row tiles (256-row tiles would split k into chunks of 256)
    ("graph_splitk_rows128_perchannel_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(200, 1024), n=512,
                                                     mode="channel")),
], ids=["graph_smallm_pergroup64_fp16_i8", "graph_largem_pergroup128_bf16_i4", "graph_largem_perchannel_bf16_i8",
        "graph_splitk_perchannel_bf16_i8", "graph_splitk_pergroup128_fp16_i4",
        "graph_splitk_rows128_perchannel_fp16_i8"])
def test_graph_replay_antiquant(name, spec):
    """A prepared call captured in a HIP graph and replayed on new inputs (copied into the
    captured buffers, with eager work and synchronisation between replays): every replay
    equals an eager call bit for bit and passes the oracle comparison."""
    import torch
    import weight_quantized_gemm_amd as W
    _announce(name)
    cases = [workloads.make_antiquant(seed=900 + i, name=f"{name}{i}", **spec) for i in range(3)]
    buf = _antiquant_tensors(cases[0])
    int4 = spec["weight"] == "int4"
    call = W.AntiquantMatmul(buf["x1"], buf["x2"], buf["scale"], buf["offset"], buf["bias"], buf["x3"],
                             cases[0].group_size, x2_int4=int4)
    call()  # eager warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for case in cases:
        new = _antiquant_tensors(case)
        for k, t in buf.items():
            if t is not None:
                t.copy_(new[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = call.out.clone()
        eager = run_antiquant(case)
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int16), eager.view(torch.int16)), case.name
        r = oracle.compare(to_f64(replayed).reshape(case.out_shape), ref_antiquant(case), case.act)
        assert r["ok"], (case.name, r)


@pytest.mark.parametrize("x1_shape,n", [((300, 256), 320), ((64, 2048), 256), ((200, 1024), 512)],
                         ids=["tiles", "splitk", "splitk_rows128"])
def test_graph_replay_w8a8(x1_shape, n):
    """The W8A8 prepared call captured and replayed on new inputs, checked like the
    anti-quant graph test (the int32 accumulator bit-exact); the second shape splits k on
    64-row tiles, the third on 128-row tiles beyond m = 128."""
    import torch
    import weight_quantized_gemm_amd as W
    _announce(f"graph_w8a8_{x1_shape}_{n}")
    cases = [workloads.make_w8a8(seed=950 + i, name=f"graph_w8a8_{i}", out="bf16", x1_shape=x1_shape, n=n)
             for i in range(3)]

    def tensors(c):
        return dict(x1=dev_tensor(c.x1, "raw"), x2=dev_tensor(c.x2, "raw"), dq=dev_tensor(c.dequant_scale, c.dequant_dtype),
                    pt=dev_tensor(c.pertoken_scale, "fp32"), bias=dev_tensor(c.bias, "raw"), x3=dev_tensor(c.x3, c.out))
    buf = tensors(cases[0])
    acc = torch.empty(cases[0].out_shape, dtype=torch.int32, device="cuda:0")
    call = W.QuantMatmul(buf["x1"], buf["x2"], buf["dq"], buf["pt"], buf["bias"], buf["x3"], acc_out=acc)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for c in cases:
        new = tensors(c)
        for k, t in buf.items():
            if t is not None:
                t.copy_(new[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, racc = ref_w8a8(c)
        assert np.array_equal(acc.cpu().numpy().astype(np.int64), racc.reshape(acc.shape))
        r = oracle.compare(to_f64(call.out).reshape(ref.shape), ref, c.out)
        assert r["ok"], (c.name, r)


@pytest.mark.parametrize("name,spec", [
    ("stream_splitk_pergroup128_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(200, 2048), n=256, mode="group",
                                               group_size=128)),
    ("stream_smallm_perchannel_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(16, 4096), n=512,
                                              mode="channel")),
], ids=["stream_splitk_pergroup128_bf16_i4", "stream_smallm_perchannel_fp16_i8"])
def test_side_stream(name, spec):
    """Calls enqueued on a non-default stream (default priority, created by torch) run every
    kernel they launch -- row-sum pass, main kernel, split-k finish -- on that stream: read
    after synchronising only that stream, the results equal calls on the default stream
    bit for bit (anti-quant, then a split W8A8 call)."""
    import torch
    import weight_quantized_gemm_amd as W
    _announce(name)
    case = workloads.make_antiquant(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    t = _antiquant_tensors(case)
    int4 = spec["weight"] == "int4"
    args = (t["x1"], t["x2"], t["scale"], t["offset"], t["bias"], t["x3"], case.group_size)
    ref = W.AntiquantMatmul(*args, x2_int4=int4)()
    side_call = W.AntiquantMatmul(*args, x2_int4=int4)
    q = workloads.make_w8a8(seed=77, name="stream_w8a8", out="bf16", x1_shape=(64, 2048), n=256)
    qa = (dev_tensor(q.x1, "raw"), dev_tensor(q.x2, "raw"), dev_tensor(q.dequant_scale, q.dequant_dtype),
          dev_tensor(q.pertoken_scale, "fp32"), dev_tensor(q.bias, "raw"), dev_tensor(q.x3, q.out))
    qref = W.QuantMatmul(*qa)()
    q_side = W.QuantMatmul(*qa)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side_call(stream=side)
    q_side(stream=side)
    side.synchronize()
    assert torch.equal(side_call.out.view(torch.int16), ref.view(torch.int16)), name
    assert torch.equal(q_side.out.view(torch.int16), qref.view(torch.int16))
    r = oracle.compare(to_f64(side_call.out).reshape(case.out_shape), ref_antiquant(case), case.act)
    assert r["ok"], (name, r)


def test_functional_form_side_stream(monkeypatch):
    """The one-shot calls with stream=<a side stream>: the output and the workspace belong to
    that stream, so once the call returns (and drops its workspace) torch's allocator does
    not hand that memory to new tensors of the current stream while the side stream's kernels
    may still use it.  A split-k call (workspace of partials), a per-group call with
    transposed parameters (workspace copies) and a split W8A8 call; results checked against
    the oracle after the current stream has written into fresh tensors of the same sizes."""
    import torch
    import weight_quantized_gemm_amd as W
    _announce("functional_side_stream")
    seen = []
    for cls_name in ("AntiquantMatmul", "QuantMatmul"):
        base = getattr(W, cls_name)

        class Spy(base):
            def __init__(self, *a, **k):
                super().__init__(*a, **k)
                seen.append((self.workspace.data_ptr(), self.workspace.numel()))
        monkeypatch.setattr(W, cls_name, Spy)
    side = torch.cuda.Stream()
    aq_cases = [workloads.make_antiquant(seed=61, name="fs_splitk", act="bf16", weight="int8", x1_shape=(64, 4096),
                                         n=512, mode="channel"),
                workloads.make_antiquant(seed=62, name="fs_xt_group", act="fp16", weight="int4", x1_shape=(300, 1024),
                                         n=256, mode="group", group_size=128, x2_transposed=True)]
    q = workloads.make_w8a8(seed=63, name="fs_w8a8", out="bf16", x1_shape=(64, 2048), n=256)
    outs, keep = [], []
    for case in aq_cases:
        outs.append(run_antiquant(case, stream=side, keep=keep))
    yq, accq = run_w8a8(q, stream=side, keep=keep)
    # the current stream now allocates and writes tensors of the workspaces' sizes
    junk = [torch.full((max(1, n),), 0x5A, dtype=torch.uint8, device="cuda:0") for _, n in seen]
    for (ptr, n), j in zip(seen, junk):
        assert n == 1 or j.data_ptr() != ptr, "a workspace was handed to the current stream"
    side.synchronize()
    torch.cuda.synchronize()
    for case, y in zip(aq_cases, outs):
        r = oracle.compare(to_f64(y).reshape(case.out_shape), ref_antiquant(case), case.act)
        assert r["ok"], (case.name, r)
    ref, racc = ref_w8a8(q)
    assert np.array_equal(accq.cpu().numpy().astype(np.int64), racc)
    assert oracle.compare(to_f64(yq).reshape(ref.shape), ref, q.out)["ok"]


W8A8_CASES = [
    ("w8a8_ragged_bf16", dict(out="bf16", x1_shape=(600, 288), n=544)),
    ("w8a8_fp16_tensor_nopt", dict(out="fp16", x1_shape=(300, 256), n=256, dequant="tensor",
                                   with_pertoken=False, with_bias=False, with_x3=False)),
    ("w8a8_bf16dq", dict(out="bf16", x1_shape=(257, 320), n=288, dequant_dtype="bf16")),
    ("w8a8_m1", dict(out="bf16", x1_shape=(1, 128), n=64)),
    ("w8a8_3d_m3", dict(out="fp16", x1_shape=(3, 1, 256), n=96)),
    ("w8a8_fp16_pt_3d", dict(out="fp16", x1_shape=(2, 130, 384), n=320)),
    ("w8a8_maxk", dict(out="bf16", x1_shape=(64, 65504), n=64)),
    ("w8a8_xt_ragged_bf16", dict(out="bf16", x1_shape=(600, 288), n=544, x2_transposed=True)),
    ("w8a8_xt_fp16_tensor_3d", dict(out="fp16", x1_shape=(2, 70, 256), n=96, dequant="tensor",
                                    with_pertoken=False, x2_transposed=True)),
    # n beyond 65535, allowed with a transposed x2 only
    ("w8a8_xt_n70016", dict(out="bf16", x1_shape=(40, 64), n=70016, x2_transposed=True)),
    # few output tiles: split k, int32 partials added by a finishing kernel (k with a 32-row
    # tail; the accumulator still bit-exact)
    ("w8a8_splitk_m64", dict(out="bf16", x1_shape=(64, 4096), n=512)),
    ("w8a8_splitk_m300_tail_xt", dict(out="fp16", x1_shape=(300, 2080), n=320, x2_transposed=True)),
    ("w8a8_splitk_m7_tensor", dict(out="bf16", x1_shape=(7, 3072), n=96, dequant="tensor", with_pertoken=False)),
    # 64-row tiles: m <= 64, and 64 < m <= 128 where 128-row tiles would split k into chunks
    # of at most 512 (two row tiles, the second ragged)
    ("w8a8_rows64_m100", dict(out="bf16", x1_shape=(100, 2048), n=512)),
    ("w8a8_rows64_m120_xt_3d", dict(out="fp16", x1_shape=(2, 60, 1024), n=768, x2_transposed=True)),
    ("w8a8_rows64_m64_xt_tensor", dict(out="bf16", x1_shape=(64, 3072), n=320, x2_transposed=True,
                                       dequant="tensor", with_pertoken=False)),
    # m > 128 with 256-row tiles that would split k into chunks of at most 512: 128-row tiles
    ("w8a8_rows128_m200_3d", dict(out="bf16", x1_shape=(2, 100, 2048), n=768)),
    ("w8a8_rows128_m256_xt", dict(out="fp16", x1_shape=(256, 1536), n=512, x2_transposed=True)),
]


@pytest.mark.parametrize("name,spec", W8A8_CASES, ids=[c[0] for c in W8A8_CASES])
def test_w8a8_parity(name, spec):
    _announce(name)
    case = workloads.make_w8a8(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    y, acc = run_w8a8(case)
    ref, racc = ref_w8a8(case)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), racc)
    r = oracle.compare(to_f64(y).reshape(ref.shape), ref, case.out)
    assert r["ok"], r


def test_page_sample_w8a8_all_ones():
    import torch
    import weight_quantized_gemm_amd as W
    _announce("page_sample_w8a8")
    d = "cuda:0"
    acc = torch.empty(32, 128, dtype=torch.int32, device=d)
    y = W.quant_matmul(torch.ones(32, 64, dtype=torch.int8, device=d),
                       torch.ones(64, 128, dtype=torch.int8, device=d),
                       torch.ones(128, dtype=torch.float32, device=d),
                       torch.ones(32, dtype=torch.float32, device=d),
                       torch.ones(128, dtype=torch.int32, device=d),
                       torch.ones(32, 128, dtype=torch.float16, device=d), acc_out=acc)
    assert torch.all(acc == 65) and torch.all(y.float() == 66)


# ---------------------------------------------------------------- full-size workloads
FULL = [n for n, s in workloads.WORKLOADS.items()]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """Every measured workload at its full size, in the configuration the benchmark times,
    compared with the oracle on every output element (and, for W8A8, the whole int32
    accumulator bit for bit)."""
    _announce(f"full:{name}")
    case = workloads.make_workload(name)
    if isinstance(case, workloads.AntiquantCase):
        check_aq(case)
    else:
        y, acc = run_w8a8(case)
        got_acc = acc.cpu().numpy().astype(np.int64)
        got = to_f64(y).reshape(-1, case.n)
        del y, acc
        ref, racc = ref_w8a8(case)
        assert np.array_equal(got_acc, racc.reshape(got_acc.shape))
        r = oracle.compare(got, ref.reshape(got.shape), case.out)
        assert r["ok"], r


# ---------------------------------------------------------------- outputs past 2^31 elements
# m = 262,181 rows of 8192 columns: 2.15e9 output elements (4.3 GB bf16), so element offsets
# in the output, the int32 accumulator and the row tiles pass the int32 range (32,800 tiles,
# no split).  Checked on sampled rows that include rows whose first element lies past 2^31;
# the rows are taken on the device before anything is copied to the host.
BIG_M, BIG_N = 262181, 8192
BIG_ROWS = [0, 1, 131072, 262143, 262144, 262145, BIG_M - 1]


def test_output_past_int32_elements_antiquant():
    import torch
    _announce("big_m_antiquant")
    case = workloads.make_antiquant(seed=2600, name="big_m", act="bf16", weight="int8",
                                    x1_shape=(BIG_M, 64), n=BIG_N, mode="channel", with_x3=False)
    rows = np.array(sorted(set(BIG_ROWS + sampled_rows(case.m).tolist())))
    y = run_antiquant(case)
    got = to_f64(y.reshape(-1, case.n)[torch.as_tensor(rows, device=y.device)])
    del y
    r = oracle.compare(got, ref_antiquant(case, rows).reshape(got.shape), case.act)
    assert r["ok"], r


def test_output_past_int32_elements_w8a8():
    import torch
    _announce("big_m_w8a8")
    case = workloads.make_w8a8(seed=2601, name="big_m_w8a8", out="bf16", x1_shape=(BIG_M, 64), n=BIG_N,
                               with_x3=False)
    rows = np.array(sorted(set(BIG_ROWS + sampled_rows(case.m).tolist())))
    y, acc = run_w8a8(case)
    idx = torch.as_tensor(rows, device=y.device)
    got, got_acc = to_f64(y.reshape(-1, case.n)[idx]), acc[idx].cpu().numpy().astype(np.int64)
    del y, acc
    ref, racc = ref_w8a8(case, rows)
    assert np.array_equal(got_acc, racc)
    r = oracle.compare(got, ref.reshape(got.shape), case.out)
    assert r["ok"], r


# ---------------------------------------------------------------- seeded sweep
def _sweep_antiquant(count=48, seed=4242, ms=(1, 2, 7, 31, 32, 33, 65, 100, 257, 300), kmax=24, prefix="sw"):
    """Random combinations of dtype, weight format, mode, layout, optional inputs and ragged
    shapes (small-m and tiled paths), each drawn from a fixed seed."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        act = str(rng.choice(["fp16", "bf16"]))
        weight = str(rng.choice(["int8", "int4", "fp8e4m3"], p=[0.45, 0.35, 0.2]))
        align = 64 if weight == "int4" else 32
        k = int(align * rng.integers(1, kmax + 1))
        n = int(align * rng.integers(1, 13))
        m = int(rng.choice(list(ms)))
        mode = "channel" if weight == "fp8e4m3" else str(rng.choice(["tensor", "channel", "group"]))
        g = 0
        if mode == "group":
            gs = [v for v in range(32, k, 32)]
            if not gs:
                mode = "channel"
            else:
                g = int(rng.choice(gs))
        lead = (m,)
        if m % 2 == 0 and m > 2 and rng.random() < 0.3:
            lead = (2, m // 2)
        spec = dict(act=act, weight=weight, x1_shape=lead + (k,), n=n, mode=mode, group_size=g,
                    with_offset=weight != "fp8e4m3" and bool(rng.random() < 0.7),
                    with_bias=bool(rng.random() < 0.6), with_x3=bool(rng.random() < 0.6),
                    channel_2d=bool(rng.random() < 0.3), x2_transposed=bool(rng.random() < 0.3))
        if weight == "fp8e4m3":
            spec["scale_dist"] = ("uniform", 2e-4, 1e-3)
        name = (f"{prefix}{i}_{act}_{weight}_{mode}{g or ''}_m{m}k{k}n{n}"
                f"{'_xt' if spec['x2_transposed'] else ''}")
        out.append((name, spec))
    return out


SWEEP = _sweep_antiquant()
# m from 33 to 200 with k up to 96 blocks of 32 (64 for int4): most of these split k, on
# the 64-, 128- and 256-row tiles
SWEEP += _sweep_antiquant(count=32, seed=4747, ms=(33, 47, 64, 65, 96, 128, 129, 200), kmax=96, prefix="swk")


@pytest.mark.parametrize("name,spec", SWEEP, ids=[c[0] for c in SWEEP])
def test_sweep_antiquant(name, spec):
    case = workloads.make_antiquant(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    check_aq(case)


def _sweep_w8a8(count=16, seed=4343):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        k = int(32 * rng.integers(1, 33))
        n = int(32 * rng.integers(1, 17))
        m = int(rng.choice([1, 5, 32, 77, 256, 300]))
        out_dt = str(rng.choice(["fp16", "bf16"]))
        dequant = str(rng.choice(["tensor", "channel"]))
        dq_dt = str(rng.choice(["fp32", "bf16"]))
        # a FLOAT16 output takes a FLOAT32 dequant scale ("aclnnQuantMatmulAllReduceV2",
        # Constraints); the draw is kept so that the other fields stay as they were
        spec = dict(out=out_dt, x1_shape=(m, k), n=n, dequant=dequant,
                    dequant_dtype=dq_dt if out_dt == "bf16" else "fp32",
                    with_bias=bool(rng.random() < 0.7), with_pertoken=bool(rng.random() < 0.7),
                    with_x3=bool(rng.random() < 0.6), x2_transposed=bool(rng.random() < 0.4))
        out.append((f"sw8_{i}_m{m}k{k}n{n}{'_xt' if spec['x2_transposed'] else ''}", spec))
    return out


SWEEP8 = _sweep_w8a8()


@pytest.mark.parametrize("name,spec", SWEEP8, ids=[c[0] for c in SWEEP8])
def test_sweep_w8a8(name, spec):
    _announce(name)
    case = workloads.make_w8a8(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    y, acc = run_w8a8(case)
    ref, racc = ref_w8a8(case)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), racc)
    r = oracle.compare(to_f64(y).reshape(ref.shape), ref, case.out)
    assert r["ok"], r
