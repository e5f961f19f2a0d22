"""CPU-only checks of the C ABI: the library loads, exports every function
include/csa.h declares, and rejects invalid arguments on the host before any
HIP call (so these run without a GPU).  Compute calls need a GPU and live in
the gpu-marked tests."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "long_context_attention_02_amd", "libcsa.so")
HEADER = os.path.join(ROOT, "include", "csa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libcsa.so not built")

CSA_OK, CSA_E_NULL, CSA_E_SHAPE, CSA_E_DTYPE, CSA_E_UNSUPPORTED, CSA_E_WORKSPACE = 0, 1, 2, 3, 4, 5


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import long_context_attention_02_amd as csa  # noqa: F401  (sets argtypes)
    return csa._lib


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"csa_compress", "csa_index_score", "csa_topk", "csa_sparse_mqa", "hca_dense_mqa"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.csa_abi_version() == 6
    for s in range(7):
        assert lib.csa_status_str(s)
    assert lib.csa_status_str(99) == b"unknown status"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_compress_validation(lib):
    args = dict(C_a=FAKE, Z_a=FAKE, C_b=FAKE, Z_b=FAKE, in_dtype=1, B=1, R=8, ibs=8 * 64, tok_base=0,
                T=8, T_len=None, c=64, m=4, overlap=1, s_begin=0, s_end=2, gamma=None, eps=1e-6, rope_dim=0,
                rope_base=1e4, pos_stride=4, pos_offset=0, E=FAKE, out_dtype=1, E_scale=None,
                obs=2 * 64, out_ring=0, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.csa_compress(*a.values())

    assert call(C_a=None) == CSA_E_NULL
    assert call(E=None) == CSA_E_NULL
    assert call(C_b=None) == CSA_E_NULL                       # overlap needs set b
    assert call(in_dtype=2) == CSA_E_DTYPE
    assert call(out_dtype=7) == CSA_E_DTYPE
    assert call(out_dtype=2) == CSA_E_NULL                    # fp8 output needs E_scale
    assert call(m=0) == CSA_E_SHAPE
    assert call(s_end=3) == CSA_E_SHAPE                       # ceil(8/4) = 2 entries only
    assert call(rope_dim=3) == CSA_E_SHAPE
    assert call(rope_dim=66) == CSA_E_SHAPE
    assert call(tok_base=1) == CSA_E_SHAPE                    # token 0 not among the rows
    assert call(R=7, ibs=7 * 64) == CSA_E_SHAPE               # token 7 missing
    assert call(c=2048, ibs=8 * 2048, obs=2 * 2048) == CSA_E_UNSUPPORTED
    assert b"csa_compress" in lib.csa_last_error()
    assert call(s_begin=1, s_end=1) == CSA_OK                 # empty range: nothing to do
    assert lib.csa_last_error() == b""
    # per-sequence token counts live on the device: the host checks the bound T only
    assert call(T_len=FAKE, s_end=3) == CSA_E_SHAPE
    assert call(T_len=FAKE, s_begin=2, s_end=2) == CSA_OK


def test_compress_batch_validation(lib):
    """Every job is checked before anything is launched; the first failing job's
    status comes back and the message names its index."""
    import long_context_attention_02_amd as csa
    good = dict(C_a=FAKE, Z_a=FAKE, C_b=FAKE, Z_b=FAKE, in_dtype=1, B=1, R=8, in_batch_stride=8 * 64,
                tok_base=0, T=8, c=64, m=4, overlap=1, s_begin=0, s_end=2, gamma=None, eps=1e-6,
                rope_dim=0, rope_base=1e4, pos_stride=4, pos_offset=0, E=FAKE, out_dtype=1,
                E_scale=None, out_batch_stride=2 * 64, out_ring=0)

    def batch(*jobs, n=None):
        arr = (csa._CompressJob * max(len(jobs), 1))()
        for q, kw in enumerate(jobs):
            arr[q] = csa._CompressJob(**dict(good, **kw))
        return lib.csa_compress_batch(arr, len(jobs) if n is None else n, None, 0, None)

    assert lib.csa_compress_batch(None, 1, None, 0, None) == CSA_E_NULL
    assert batch({}, n=0) == CSA_E_SHAPE
    assert batch(*([{}] * 9)) == CSA_E_SHAPE                  # at most CSA_COMPRESS_MAX_JOBS
    assert batch({}, {"m": 0}) == CSA_E_SHAPE
    assert b"job 1" in lib.csa_last_error()
    assert batch({"out_dtype": 2}, {"s_end": 3}) == CSA_E_NULL   # job 0 fails first
    assert b"job 0" in lib.csa_last_error()
    assert batch({"c": 2048, "in_batch_stride": 8 * 2048, "out_batch_stride": 2 * 2048}) == CSA_E_UNSUPPORTED
    # only empty ranges: valid, nothing launched
    assert batch({"s_begin": 1, "s_end": 1}, {"s_begin": 0, "s_end": 0}) == CSA_OK
    assert lib.csa_last_error() == b""


def test_compress_batch_workspace(lib):
    """The channel-split path's workspace: HCA-like entries (128 candidates, 512
    channels) in a small launch take 8 slices each; slice sums (a 256-byte
    aligned region), then rows.  Too small a workspace is refused before any
    launch; jobs of few candidates or many entries need none."""
    import long_context_attention_02_amd as csa
    hca = dict(C_a=FAKE, Z_a=FAKE, C_b=None, Z_b=None, in_dtype=1, B=4, R=128, in_batch_stride=128 * 512,
               tok_base=8191 * 128, T=8192 * 128, c=512, m=128, overlap=0, s_begin=8191, s_end=8192, gamma=None,
               eps=1e-6, rope_dim=64, rope_base=1e4, pos_stride=128, pos_offset=0, E=FAKE, out_dtype=1,
               E_scale=None, out_batch_stride=8192 * 512, out_ring=0)
    win = dict(hca, m=1, s_begin=0, s_end=1, R=1, in_batch_stride=512, tok_base=0, T=1, pos_stride=1)

    def arr(*jobs):
        a = (csa._CompressJob * len(jobs))()
        for q, kw in enumerate(jobs):
            a[q] = csa._CompressJob(**kw)
        return a

    slots = 4
    need = 256 + slots * 512 * 4            # 4 x 8 slice sums, 4 rows of 512 floats
    assert lib.csa_compress_workspace_size(arr(win, hca), 2) == need
    assert lib.csa_compress_workspace_size(arr(win), 1) == 0                       # one candidate
    many = dict(hca, s_begin=8000, tok_base=8000 * 128, R=192 * 128, in_batch_stride=192 * 128 * 512)
    assert lib.csa_compress_workspace_size(arr(dict(many, B=1)), 1) > 0              # 192 items
    assert lib.csa_compress_workspace_size(arr(many), 1) == 0                        # 4 x 192 > 256 items
    assert lib.csa_compress_workspace_size(arr(dict(hca, m=0)), 1) == 0            # invalid: counts nothing
    assert lib.csa_compress_batch(arr(win, hca), 2, FAKE, need - 1, None) == CSA_E_WORKSPACE


def test_index_score_validation(lib):
    base = [FAKE, 1, FAKE, FAKE, 1, None, FAKE, 2, 1, 64, 128, 1000, 4, FAKE, None]

    def call(**kw):
        a = list(base)
        names = ["q", "qd", "w", "K", "kd", "Ks", "pos", "B", "Tq", "H", "dI", "N", "m", "out", "st"]
        for k_, v in kw.items():
            a[names.index(k_)] = v
        return lib.csa_index_score(*a)

    assert call(q=None) == CSA_E_NULL
    assert call(out=None) == CSA_E_NULL
    assert call(kd=2) == CSA_E_NULL                           # fp8 keys need K_scale
    assert call(qd=0) == CSA_E_DTYPE                          # f32 queries with bf16 keys
    assert call(kd=0) == CSA_E_DTYPE
    assert call(qd=2) == CSA_E_DTYPE
    assert call(m=0) == CSA_E_SHAPE
    assert call(N=0) == CSA_E_SHAPE
    assert call(H=65) == CSA_E_UNSUPPORTED
    assert call(dI=512) == CSA_E_UNSUPPORTED


def test_decode_front_validation(lib):
    """csa_decode_front checks its jobs and the indexer's arguments as the two
    separate calls do, then refuses (CSA_E_UNSUPPORTED, nothing launched) what
    the one-launch path does not cover."""
    import long_context_attention_02_amd as csa
    B, H, dI, N = 2, 64, 128, 4096
    # fake buffers far apart: keys (1 MiB), their scales, the KV rows and the window ring
    KEYS, SCALES, ROWS = FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24)
    win = dict(C_a=FAKE, Z_a=None, C_b=None, Z_b=None, in_dtype=1, B=B, R=1, in_batch_stride=512, tok_base=4 * N,
               T=4 * N + 1, c=512, m=1, overlap=0, s_begin=4 * N, s_end=4 * N + 1, gamma=FAKE, eps=1e-6,
               rope_dim=64, rope_base=1e4, pos_stride=1, pos_offset=0, E=ROWS, out_dtype=1,
               E_scale=None, out_batch_stride=128 * 512, out_ring=128)
    key = dict(C_a=FAKE, Z_a=FAKE, C_b=FAKE, Z_b=FAKE, in_dtype=1, B=B, R=8, in_batch_stride=8 * dI,
               tok_base=4 * (N - 2), T=4 * N, c=dI, m=4, overlap=1, s_begin=N - 1, s_end=N, gamma=None,
               eps=1e-6, rope_dim=0, rope_base=1e4, pos_stride=4, pos_offset=0, E=KEYS, out_dtype=2,
               E_scale=SCALES, out_batch_stride=N * dI, out_ring=0)

    def call(jobs=(win, key), n=None, N_=N, kd=2, Ks=SCALES, K=KEYS, H_=H, q=FAKE):
        arr = (csa._CompressJob * max(len(jobs), 1))()
        for i, kw in enumerate(jobs):
            arr[i] = csa._CompressJob(**kw)
        return lib.csa_decode_front(ctypes.cast(arr, ctypes.c_void_p), len(jobs) if n is None else n, q, 1, FAKE,
                                    K, kd, Ks, FAKE, B, H_, dI, N_, 4, FAKE, None)

    assert lib.csa_decode_front(None, 1, FAKE, 1, FAKE, KEYS, 2, SCALES, FAKE, B, H, dI, N, 4, FAKE,
                                None) == CSA_E_NULL
    assert call(n=0) == CSA_E_SHAPE
    assert call(jobs=[win] * 5) == CSA_E_SHAPE                                  # at most 4 jobs
    assert call(jobs=(win, dict(key, m=0))) == CSA_E_SHAPE
    assert b"job 1" in lib.csa_last_error()
    assert call(jobs=(win, dict(key, s_end=N - 1))) == CSA_E_SHAPE              # a job with no entries
    assert call(q=None) == CSA_E_NULL
    assert call(Ks=None) == CSA_E_NULL                                           # fp8 keys need K_scale
    assert call(H_=65) == CSA_E_UNSUPPORTED
    # not covered by the one-launch path
    assert call(N_=N + 32) == CSA_E_UNSUPPORTED                                 # N_cap % 64
    assert call(jobs=(win,)) == CSA_E_UNSUPPORTED and b"no compress job writes K_I" in lib.csa_last_error()
    early = dict(key, tok_base=4 * (N - 101), T=4 * (N - 99), s_begin=N - 100, s_end=N - 99)
    assert call(jobs=(win, early)) == CSA_E_UNSUPPORTED                           # not the last 64 rows
    assert call(jobs=(win, dict(key, out_dtype=1, E_scale=None))) == CSA_E_UNSUPPORTED   # key format != k_dtype
    nine = dict(win, m=9, R=9, in_batch_stride=9 * 512, tok_base=0, T=9, s_begin=0, s_end=1, pos_stride=9)
    assert call(jobs=(nine, key)) == CSA_E_UNSUPPORTED                            # 9 candidates per entry
    assert call(jobs=(dict(win, in_dtype=0, in_batch_stride=512), key)) == CSA_E_UNSUPPORTED   # f32 inputs
    assert call(jobs=(win, key, key)) == CSA_E_UNSUPPORTED                       # two jobs write the keys
    assert call(K=KEYS + 8, jobs=(win, dict(key, E=KEYS + 8))) == CSA_E_UNSUPPORTED   # 16-byte alignment
    assert call(kd=3) == CSA_E_UNSUPPORTED                                       # MXFP4 keys
    # another job writing inside the key rows (or their scales) would race with the indexer
    assert call(jobs=(dict(win, E=KEYS + 4096), key)) == CSA_E_UNSUPPORTED
    assert b"K_I or K_scale" in lib.csa_last_error()
    assert call(jobs=(dict(key, E=ROWS, E_scale=SCALES + 64), key)) == CSA_E_UNSUPPORTED


def test_topk_validation_and_workspace(lib):
    def call(k=16, ws=None, wsb=0, N=1000, B=1, Tq=1, I=FAKE, idx=FAKE):
        return lib.csa_topk(I, FAKE, B, Tq, N, 4, k, idx, None, ws, wsb, None)

    assert call(I=None) == CSA_E_NULL
    assert call(idx=None) == CSA_E_NULL
    assert call(k=0) == CSA_E_SHAPE
    assert call(k=2049) == CSA_E_SHAPE
    need = lib.csa_topk_workspace_size(16, 1, 262144, 1024)
    # 16 chunks of 16k per row, each keeping its 127 largest keys (a list of 128 slots)
    # and one threshold key: 1024 / 16 = 64 of the row's top-k per chunk on average
    assert need == 16 * 16 * (128 + 1) * 8
    assert lib.csa_topk_workspace_size(1, 16384, 32768, 1024) == 0
    assert call(k=1024, N=262144, B=16, wsb=need - 1, ws=FAKE) == CSA_E_WORKSPACE
    assert call(k=1024, N=262144, B=16) == CSA_E_WORKSPACE


def test_mqa_validation(lib):
    def sparse(**kw):
        a = dict(q=FAKE, g=None, eps=1e-6, E=FAKE, Es=None, N=100, idx=FAKE, k=16, W=FAKE, Ws=None, Wc=16,
                 nw=16, sink=None, pos=FAKE, B=1, Tq=1, nh=16, d=128, r=64, base=1e4, scale=0.1, dt=1,
                 out=FAKE, ws=None, wsb=0, st=None)
        a.update(kw)
        return lib.csa_sparse_mqa(*a.values())

    assert sparse(q=None) == CSA_E_NULL
    assert sparse(idx=None) == CSA_E_NULL
    assert sparse(W=None) == CSA_E_NULL
    assert sparse(Wc=8) == CSA_E_SHAPE                        # ring smaller than the window
    assert sparse(dt=2) == CSA_E_DTYPE
    assert sparse(d=127, r=0) == CSA_E_SHAPE
    assert sparse(r=130) == CSA_E_SHAPE
    assert sparse(k=0) == CSA_E_SHAPE
    # a split decode query needs workspace
    # 1152 slots in ranges of 192: 6 split partials per (query, head), each d fp16
    # outputs and a float record (max, sum, 1 / scale, 0); above 1536 slots the
    # ranges hold 160
    assert lib.csa_mqa_workspace_size(4, 1, 64, 512, 8192 + 128) == 4 * 52 * 64 * (512 * 2 + 16)
    assert lib.csa_mqa_workspace_size(16, 1, 128, 512, 1024 + 128) == 16 * 6 * 128 * (512 * 2 + 16)
    assert sparse(k=1024, nh=128, d=512, B=16) == CSA_E_WORKSPACE
    need = lib.csa_mqa_workspace_size(16, 1, 128, 512, 1024 + 128)
    assert sparse(k=1024, nh=128, d=512, B=16, ws=FAKE + 4, wsb=need + 16) == CSA_E_WORKSPACE
    assert b"16-byte aligned" in lib.csa_last_error()
    # prefill (16 or more queries per sequence): one range of up to 2,048 slots per query
    assert lib.csa_mqa_workspace_size(1, 16384, 128, 512, 1024 + 128) == 0
    assert lib.csa_mqa_workspace_size(1, 16, 32, 128, 2300 + 64) == 16 * 2 * 32 * (128 * 2 + 16)
    # the generic path caps the key count
    assert sparse(dt=0, k=9000) == CSA_E_UNSUPPORTED
    # mixed rows: row scales required; d = 512 and rope_dim = 64 only
    assert sparse(dt=4) == CSA_E_NULL
    assert sparse(dt=4, Es=FAKE) == CSA_E_NULL                # window rows need W_scale
    assert sparse(dt=4, Es=FAKE, Ws=FAKE) == CSA_E_UNSUPPORTED   # d = 128
    assert sparse(dt=4, Es=FAKE, Ws=FAKE, d=512, r=32) == CSA_E_UNSUPPORTED
    assert sparse(dt=5) == CSA_E_DTYPE

    def dense(**kw):
        a = dict(q=FAKE, g=None, eps=1e-6, E=FAKE, Es=None, N=100, m=0, W=FAKE, Ws=None, Wc=16, nw=16,
                 sink=None, pos=FAKE, B=1, Tq=1, nh=16, d=128, r=64, base=1e4, scale=0.1, dt=1, out=FAKE,
                 ws=None, wsb=0, st=None)
        a.update(kw)
        return lib.hca_dense_mqa(*a.values())

    assert dense() == CSA_E_SHAPE                             # m = 0
    assert dense(m=128, out=None) == CSA_E_NULL


def test_grouped_out_proj_validation(lib):
    def call(**kw):
        a = dict(o=FAKE, W1=FAKE, W2=FAKE, y=FAKE, out=FAKE, T=16, n_h=128, c=512, g=16, d_g=1024,
                 d=7168, ws=None, wsb=0, st=None)
        a.update(kw)
        return lib.csa_grouped_out_proj(*a.values())

    assert call(o=None) == CSA_E_NULL
    assert call(g=3) == CSA_E_SHAPE                           # n_h c not a multiple of groups
    assert call(d_g=1001) == CSA_E_UNSUPPORTED                # groups d_g not a multiple of 64
    assert call(o=FAKE + 2) == CSA_E_UNSUPPORTED              # unaligned
    need = lib.csa_out_proj_workspace_size(16, 128, 512, 16, 1024, 7168)
    assert need > 0                                           # few rows split the contraction
    assert call() == CSA_E_WORKSPACE
    assert lib.csa_out_proj_workspace_size(16384, 128, 512, 16, 1024, 7168) == 0


def test_cache_append_validation(lib):
    def call(**kw):
        a = dict(B=2, T0=FAKE, n=1, c=512, dI=128, m=4, mh=128, **{f"p{i}": FAKE for i in range(11)},
                 tail=FAKE, E=FAKE, K=FAKE, Ks=None, kd=1, Nc=100, H=FAKE, Nh=10, W=FAKE, Wc=128, g=None,
                 eps=1e-6, r=64, base=1e4, st=None)
        a.update(kw)
        return lib.csa_cache_append(*a.values())

    assert call(T0=None) == CSA_E_NULL
    assert call(p3=None) == CSA_E_NULL
    assert call(kd=2) == CSA_E_NULL                           # fp8 keys need K_scale
    assert call(kd=0) == CSA_E_DTYPE
    assert call(mh=4) == CSA_E_UNSUPPORTED                    # lcm(4, 4) < 2 m: the ring is too short
    assert call(c=500) == CSA_E_UNSUPPORTED
    assert call(p0=FAKE + 8) == CSA_E_UNSUPPORTED             # 16-byte alignment
    assert call(r=65) == CSA_E_SHAPE
    assert call(n=0) == CSA_E_SHAPE


def _kernel_scratch_sizes():
    """(kernel, private segment bytes) of every gfx950 kernel in libcsa.so, read from
    the code objects the build embedded (one offload bundle per source file)."""
    import shutil
    import subprocess
    import tempfile
    llvm = "/opt/rocm/llvm/bin"
    tools = [os.path.join(llvm, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(shutil.which(t) or os.path.exists(t) for t in tools):
        pytest.skip("ROCm LLVM tools not found")
    out = []
    with tempfile.TemporaryDirectory() as td:
        fb = os.path.join(td, "fatbin")
        subprocess.run([tools[0], "--dump-section", f".hip_fatbin={fb}", LIB, os.path.join(td, "copy.so")],
                       check=True, capture_output=True)
        data = open(fb, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts, i = [], data.find(magic)
        while i >= 0:
            starts.append(i)
            i = data.find(magic, i + 1)
        for n, a in enumerate(starts):
            # a bundle's header gives its entries' offsets: everything from its start will do
            part, co = os.path.join(td, f"b{n}"), os.path.join(td, f"b{n}.co")
            open(part, "wb").write(data[a:])
            r = subprocess.run([tools[1], "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                                f"--input={part}", f"--output={co}", "--unbundle"], capture_output=True)
            if r.returncode != 0:
                continue
            notes = subprocess.run([tools[2], "--notes", co], capture_output=True, text=True).stdout
            name = None
            for ln in notes.splitlines():
                m = re.match(r"\s+\.name:\s+(\S+)", ln)
                if m:
                    name = m.group(1)
                m = re.match(r"\s+\.private_segment_fixed_size:\s+(\d+)", ln)
                if m and name:
                    out.append((name, int(m.group(1))))
                    name = None
    return out


def test_no_kernel_spills_to_scratch():
    """Register spills to scratch memory have made kernels here many times slower
    (a wave-per-entry compressor went from 0.044 to 0.5 ms); every kernel of the
    library must fit its registers.  The one exception: the streaming attention
    kernel at d = 512 with two 16-head tiles per wave, whose 256 accumulator
    registers leave a few prologue values (at most 64 bytes) to scratch, none in
    the loop."""
    sizes = _kernel_scratch_sizes()
    assert len(sizes) >= 100, sizes
    allowed = re.compile(r"mqa_decode_kernelILi512ELb[01]ELi\d+ELi\d+ELi2ELb[01]EE")
    spilled = [(n, s) for n, s in sizes if s > 0 and not (allowed.search(n) and s <= 64)]
    assert not spilled, spilled
