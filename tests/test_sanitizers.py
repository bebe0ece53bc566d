"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/ttt_oracle.c) is compiled with
  -fsanitize=address,undefined into a temporary directory and the oracle
  pins (tests/test_oracle_linear.py, tests/test_oracle_mlp.py, the heavy
  full-workload pin left out) run against it in a subprocess, with the ASan
  runtime preloaded into the Python interpreter.
* The C ABI's host-side argument checks (csrc/ttt_validate.cpp, no HIP
  dependency) are compiled with g++ and the same sanitizers together with a
  small driver that walks the error paths (null pointers, shapes, flags,
  aliasing, workspace sizes and alignment, the no-allocation scratch limit,
  sizes near the 64-bit limits) and the argument fill of valid calls.
Any sanitizer report fails the test (errors are fatal: halt_on_error)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_rnn_ttt_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _no_report(out):
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "libttt_oracle_san.so"
    subprocess.check_call(["gcc", "-std=c11", "-fPIC", "-shared"] + SAN +
                          ["-o", str(lib), os.path.join(ROOT, "oracle", "ttt_oracle.c"), "-lm",
                           "-lpthread"])
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    env = dict(os.environ, TTT_ORACLE_LIB_OVERRIDE=str(lib), LD_PRELOAD=asan, **ENV)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-k", "not ill_conditioned", "tests/test_oracle_linear.py",
                        "tests/test_oracle_mlp.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    _no_report(out)
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out


DRIVER = r'''
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include "ttt_validate.hpp"

static int fails = 0;
#define EXPECT(x, want) do { ttt_status s_ = (x); if (s_ != (want)) { \
  std::printf("line %d: got %d want %d\n", __LINE__, (int)s_, (int)(want)); ++fails; } } while (0)

// fake, distinct device addresses (never dereferenced)
static void* A(int i) { return reinterpret_cast<void*>((uintptr_t(1) << 40) + uintptr_t(i) * (uintptr_t(1) << 36)); }
static float* F(int i) { return static_cast<float*>(A(i)); }

static ttt_params P(int B = 2, int H = 3, int T = 100, int d = 64, int mb = 16, int io = TTT_BF16,
                    unsigned flags = 0, float eps = 1e-6f, int s0 = 0) {
  ttt_params p;
  p.B = B; p.H = H; p.T = T; p.d = d; p.mini_batch = mb; p.io_dtype = io; p.flags = flags;
  p.ln_eps = eps; p.state0_per_batch = s0;
  return p;
}

static ttt_status lin(const ttt_params* p, void* q = A(1), void* z = A(8), float* wo = F(9),
                      const float* w0 = F(5)) {
  tttk::LinearArgs a;
  return tttv::linear_forward(p, q, A(2), A(3), F(4), w0, F(6), F(7), z, wo, nullptr, 0, &a);
}

int main() {
  ttt_params p = P();
  EXPECT(lin(nullptr), TTT_ERR_NULL);
  EXPECT(lin(&p), TTT_OK);
  EXPECT(lin(&p, nullptr), TTT_ERR_NULL);
  EXPECT(lin(&p, A(1), A(1)), TTT_ERR_ALIAS);             // z == q
  EXPECT(lin(&p, A(1), A(8), F(5)), TTT_ERR_ALIAS);       // w_out == w0, shared W0
  ttt_params s1 = P(2, 3, 100, 64, 16, TTT_BF16, 0, 1e-6f, 1);
  EXPECT(lin(&s1, A(1), A(8), F(5)), TTT_OK);             // in-place resume
  ttt_params bad[] = {P(0), P(2, 0), P(2, 3, 0), P(2, 3, (1 << 22) + 1), P(2, 3, 100, 32),
                      P(2, 3, 100, 64, 8), P(2, 3, 100, 64, 16, 7), P(2, 3, 100, 64, 16, TTT_BF16, 8),
                      P(2, 3, 100, 64, 16, TTT_BF16, 0, -1.f), P(2, 3, 100, 64, 16, TTT_BF16, 0, 1e-6f, 2),
                      P(46341, 46341), P(1 << 20, 1 << 10, 1 << 22)};
  const ttt_status want[] = {TTT_ERR_SHAPE, TTT_ERR_SHAPE, TTT_ERR_SHAPE, TTT_ERR_SHAPE,
                             TTT_ERR_UNSUPPORTED, TTT_ERR_UNSUPPORTED, TTT_ERR_ARG, TTT_ERR_ARG,
                             TTT_ERR_ARG, TTT_ERR_ARG, TTT_ERR_SHAPE, TTT_ERR_SHAPE};
  for (unsigned i = 0; i < sizeof(want) / sizeof(want[0]); ++i) EXPECT(lin(&bad[i]), want[i]);
  {  // valid fill
    tttk::LinearArgs a;
    ttt_params pm = P(2, 3, 100, 64, 64);
    EXPECT(tttv::linear_forward(&pm, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9),
                                nullptr, 0, &a), TTT_OK);
    if (a.T != 100 || a.tiles_per_mb != 4 || a.split != 0 || a.bases) ++fails;
  }
  // split launch: workspace size, alignment, overlap, in-place
  const uint64_t need = tttv::split_layout(&p).total;
  {
    tttk::LinearArgs a;
    EXPECT(tttv::linear_split(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9), nullptr,
                              need, &a), TTT_ERR_NULL);
    EXPECT(tttv::linear_split(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9), A(20),
                              need - 1, &a), TTT_ERR_SHAPE);
    EXPECT(tttv::linear_split(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9),
                              static_cast<char*>(A(20)) + 128, need, &a), TTT_ERR_ARG);
    EXPECT(tttv::linear_split(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9), A(8),
                              need, &a), TTT_ERR_ALIAS);
    EXPECT(tttv::linear_split(&s1, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(5), A(20),
                              need, &a), TTT_ERR_ALIAS);
    EXPECT(tttv::linear_split(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9), A(20),
                              need, &a), TTT_OK);
    if (a.split != 1 || reinterpret_cast<char*>(a.ws_flags) != static_cast<char*>(A(20)) ||
        reinterpret_cast<char*>(a.ws_g) - reinterpret_cast<char*>(a.ws_flags) !=
            (int64_t)tttv::split_layout(&p).stream_offset) ++fails;
  }
  {  // the no-allocation launch's scratch limit
    tttk::LinearArgs a;
    const uint64_t cap = 128ull << 20;
    ttt_params fit = P(1, 32, 10912), over = P(1, 32, 10913);
    EXPECT(tttv::linear_split_noalloc(&fit, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9),
                                      cap, &a), TTT_OK);
    EXPECT(tttv::linear_split_noalloc(&over, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8),
                                      F(9), cap, &a), TTT_ERR_TOO_LARGE);
  }
  {  // forward with saved bases
    tttk::LinearArgs a;
    const uint64_t bw = tttv::backward_layout(&p).total;
    EXPECT(tttv::linear_forward_save(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9),
                                     A(20), bw - 1, &a), TTT_ERR_SHAPE);
    EXPECT(tttv::linear_forward_save(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), F(9),
                                     A(20), bw, &a), TTT_OK);
    if (a.bases != F(20)) ++fails;
  }
  {  // streaming steps
    tttk::DecodeArgs a;
    ttt_params d1 = P(2, 3, 1);
    EXPECT(tttv::linear_decode(&d1, 0, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), A(9), &a),
           TTT_OK);
    EXPECT(tttv::linear_decode(&p, 0, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), A(9), &a),
           TTT_ERR_SHAPE);
    EXPECT(tttv::linear_decode(&d1, 16, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), A(9), &a),
           TTT_ERR_ARG);
    EXPECT(tttv::linear_decode(&d1, 0, A(1), A(2), A(3), F(4), F(5), F(5), F(7), F(8), A(9), &a),
           TTT_ERR_ALIAS);
    tttk::CompactArgs c;
    EXPECT(tttv::linear_decode_compact(&d1, 3, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8),
                                       A(9), &c), TTT_OK);
    ttt_params d65 = P(2, 3, 1, 64, 65);
    EXPECT(tttv::linear_decode_compact(&d65, 3, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8),
                                       A(9), &c), TTT_ERR_UNSUPPORTED);
    tttk::MlpDecodeArgs m;
    EXPECT(tttv::mlp_decode(&d1, 256, 0, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9),
                            F(10), F(11), F(12), F(13), F(14), A(15), &m), TTT_OK);
    EXPECT(tttv::mlp_decode(&d1, 128, 0, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9),
                            F(10), F(11), F(12), F(13), F(14), A(15), &m), TTT_ERR_UNSUPPORTED);
    EXPECT(tttv::mlp_decode(&d1, 256, 0, A(1), A(2), A(3), F(4), F(5), F(6), F(5), F(8), F(9),
                            F(10), F(11), F(12), F(13), F(14), A(15), &m), TTT_ERR_ALIAS);
    tttk::MlpCompactArgs mc;
    EXPECT(tttv::mlp_decode_compact(&d1, 256, 5, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8),
                                    F(9), F(10), F(11), A(12), &mc), TTT_OK);
  }
  {  // backward
    tttk::BackwardArgs a;
    const uint64_t bw = tttv::backward_layout(&p).total;
    EXPECT(tttv::linear_backward(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), nullptr,
                                 A(9), A(10), A(11), F(12), F(13), F(14), F(15), A(20), bw, &a),
           TTT_OK);
    EXPECT(tttv::linear_backward(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), nullptr,
                                 A(9), A(10), A(11), F(12), F(13), F(14), F(15), A(20), bw - 1, &a),
           TTT_ERR_SHAPE);
    EXPECT(tttv::linear_backward(&p, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), nullptr,
                                 A(9), A(9), A(11), F(12), F(13), F(14), F(15), A(20), bw, &a),
           TTT_ERR_ALIAS);
    ttt_params saved = P(2, 3, 100, 64, 16, TTT_BF16, TTT_BASES_SAVED);
    EXPECT(tttv::linear_backward(&saved, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), nullptr,
                                 A(9), A(10), A(11), F(12), F(13), F(14), F(15), A(20), bw, &a),
           TTT_OK);
    if (a.bases_saved != 1) ++fails;
    ttt_params mb32 = P(2, 3, 100, 64, 32, TTT_BF16, 0);
    EXPECT(tttv::linear_backward(&mb32, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), nullptr,
                                 A(9), A(10), A(11), F(12), F(13), F(14), F(15), A(20), bw, &a),
           TTT_OK);
    if (a.tiles_per_mb != 2) ++fails;
    ttt_params mb24 = P(2, 3, 100, 64, 24, TTT_BF16, 0);
    EXPECT(tttv::linear_backward(&mb24, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8), nullptr,
                                 A(9), A(10), A(11), F(12), F(13), F(14), F(15), A(20), bw, &a),
           TTT_ERR_UNSUPPORTED);
    ttt_params saved32 = P(2, 3, 100, 64, 32, TTT_BF16, TTT_BASES_SAVED);
    EXPECT(tttv::linear_backward(&saved32, A(1), A(2), A(3), F(4), F(5), F(6), F(7), A(8),
                                 nullptr, A(9), A(10), A(11), F(12), F(13), F(14), F(15), A(20),
                                 bw, &a), TTT_ERR_UNSUPPORTED);
  }
  {  // MLP backward
    tttk::MlpBackwardArgs m;
    const uint64_t need = tttv::mlp_backward_workspace_bytes(&p);
    EXPECT(tttv::mlp_backward(&p, 256, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9),
                              F(10), A(11), nullptr, nullptr, nullptr, nullptr, A(12), A(13),
                              A(14), F(15), F(16), F(17), F(18), F(19), F(21), F(22), A(20),
                              need, &m), TTT_OK);
    EXPECT(tttv::mlp_backward(&p, 256, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9),
                              F(10), A(11), nullptr, nullptr, nullptr, nullptr, A(12), A(13),
                              A(14), F(15), F(16), F(17), F(18), F(19), F(21), F(22), A(20),
                              need - 1, &m), TTT_ERR_SHAPE);
    EXPECT(tttv::mlp_backward(&p, 256, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9),
                              F(10), A(11), nullptr, nullptr, nullptr, nullptr, A(12), A(12),
                              A(14), F(15), F(16), F(17), F(18), F(19), F(21), F(22), A(20),
                              need, &m), TTT_ERR_ALIAS);
  }
  {  // input side
    tttk::InputArgs in;
    EXPECT(tttv::input_projection(&p, 128, A(1), A(2), F(3), 0.01f, A(4), A(5), A(6), F(7), &in),
           TTT_OK);
    if (in.D != 128 || in.H != 3) ++fails;
    EXPECT(tttv::input_projection(&p, 100, A(1), A(2), F(3), 0.01f, A(4), A(5), A(6), F(7), &in),
           TTT_ERR_UNSUPPORTED);
    EXPECT(tttv::input_projection(&p, 128, A(1), A(2), F(3), 0.0f, A(4), A(5), A(6), F(7), &in),
           TTT_ERR_ARG);
    EXPECT(tttv::input_projection(&p, 128, A(1), A(2), F(3), 0.01f, A(1), A(5), A(6), F(7), &in),
           TTT_ERR_ALIAS);
    EXPECT(tttv::input_projection(&p, 128, A(1), A(2), F(3), 0.01f, A(4), nullptr, A(6), F(7),
                                  &in), TTT_ERR_NULL);
  }
  {  // MLP forward
    tttk::MlpArgs a;
    EXPECT(tttv::mlp_forward(&p, 256, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9), F(10),
                             A(11), F(12), F(13), F(14), F(15), &a), TTT_OK);
    EXPECT(tttv::mlp_forward(&p, 256, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9), F(10),
                             A(11), F(12), nullptr, F(14), F(15), &a), TTT_ERR_NULL);
    EXPECT(tttv::mlp_forward(&p, 0, A(1), A(2), A(3), F(4), F(5), F(6), F(7), F(8), F(9), F(10),
                             A(11), F(12), F(13), F(14), F(15), &a), TTT_ERR_SHAPE);
  }
  if (fails) { std::printf("%d failed\n", fails); return 1; }
  std::printf("validation ok\n");
  return 0;
}
'''


def test_abi_validation_under_sanitizers(tmp_path):
    drv = tmp_path / "driver.cpp"
    drv.write_text(DRIVER)
    exe = tmp_path / "validate_san"
    subprocess.check_call(["g++", "-std=c++17", "-Wall"] + SAN +
                          ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(exe),
                           os.path.join(CSRC, "ttt_validate.cpp"), str(drv)])
    r = subprocess.run([str(exe)], env=dict(os.environ, **ENV), capture_output=True, text=True,
                       timeout=120)
    out = r.stdout + r.stderr
    _no_report(out)
    assert r.returncode == 0 and "validation ok" in out, out[-4000:]
