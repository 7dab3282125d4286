// abi_driver.cpp -- the host side of the C ABI (csrc/kda_api.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU: the kernel
// launchers are replaced by recording stubs, so every entry point runs its
// argument validation, workspace layout and launch sequencing on the host.
// Checks that valid calls reach the right launchers with a workspace layout
// that fits the buffer, that invalid calls are refused before any launch with
// the documented status, and that a refused launch becomes
// KDA_ERROR_LAUNCH_FAILED.  Built and run by tests/test_sanitizers.py; exit
// status 0 when every check holds.  Device pointers are never dereferenced
// on the host, so aligned dummy addresses stand in for them.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda.h"
#include "kda_internal.hpp"

namespace {
struct Record {
  int intra = 0, inter = 0, epilogue = 0, check_cu = 0, decode = 0, bwd = 0, table = 0;
  int64_t table_entries = 0;
  const int4 *tab = nullptr;
  kda::FwdArgs fwd{};
  kda::BwdArgs bwdargs{};
  int64_t epi_rows = 0;
  int decode_batch = 0;
};
Record rec;
hipError_t launch_result = hipSuccess;
int failures = 0;

void check(bool ok, const char *what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAIL (line %d): %s\n", line, what);
    ++failures;
  }
}
#define CHECK(x) check((x), #x, __LINE__)

int launches() {
  return rec.intra + rec.inter + rec.epilogue + rec.check_cu + rec.decode + rec.bwd + rec.table;
}
void reset() { rec = Record(); launch_result = hipSuccess; }

void *dev(uintptr_t i) { return reinterpret_cast<void *>((uintptr_t)0x100000 + 0x1000 * i); }
}  // namespace

namespace kda {
int device_cus() { return 256; }
hipError_t launch_intra(const FwdArgs &a, kda_dtype) { ++rec.intra; rec.fwd = a; return launch_result; }
hipError_t launch_inter(const FwdArgs &a, kda_dtype) { ++rec.inter; rec.fwd = a; return launch_result; }
hipError_t launch_check_cu(const int *, int, int64_t, int *, hipStream_t) {
  ++rec.check_cu;
  return launch_result;
}
hipError_t launch_chunk_table(const int *, int, int64_t, int, int64_t max_chunks, int4 *tab,
                              int *, const OptArgs &, hipStream_t) {
  ++rec.table;
  rec.table_entries = max_chunks;
  rec.tab = tab;
  return launch_result;
}
hipError_t launch_bwd(const BwdArgs &a, kda_dtype) { ++rec.bwd; rec.bwdargs = a; return launch_result; }
hipError_t launch_out_epilogue(void *, const OptArgs &, int64_t rows, int, kda_dtype, hipStream_t) {
  ++rec.epilogue;
  rec.epi_rows = rows;
  return launch_result;
}
hipError_t launch_decode(const void *, const void *, const void *, const void *, const float *,
                         const OptArgs &, float *, void *, int batch, int, int, kda_dtype,
                         hipStream_t) {
  ++rec.decode;
  rec.decode_batch = batch;
  return launch_result;
}
}  // namespace kda

namespace {

struct Fwd {
  int64_t T = 4096;
  int32_t N = 2, H = 8, d = 128, C = 64;
  kda_dtype dt = KDA_DTYPE_BF16;
  const void *q = dev(1), *k = dev(2), *v = dev(3);
  const void *g = dev(4);
  const float *beta = static_cast<const float *>(dev(5));
  const int32_t *cu = nullptr;
  const float *s0 = nullptr;
  float *sf = static_cast<float *>(dev(7));
  void *o = dev(8);
  void *ws = dev(9);
  size_t ws_bytes = 0;
  const kda_options *opt = nullptr;
  uint32_t stages = 3;

  void fit() { ws_bytes = kda_fwd_chunked_workspace_size(T, N, H, d, d, C, dt); }
  kda_status run() const {
    return kda_fwd_chunked_ex(opt, stages, q, k, v, g, beta, cu, N, T, H, d, d, C, dt, s0, sf, o,
                              ws, ws_bytes, nullptr);
  }
};

void layout_fits(const kda::FwdArgs &a, size_t ws_bytes) {
  const kda::FwdLayout &L = a.lay;
  CHECK(L.total <= ws_bytes);
  const size_t offs[] = {L.seq_first, L.chunk_tab, L.qt, L.w, L.ut, L.ket, L.p, L.gam};
  for (size_t off : offs) {
    CHECK(off % 256 == 0);
    CHECK(off < L.total || (off == L.total && a.total_tokens == 0));
  }
  CHECK(L.seq_first < L.chunk_tab && L.chunk_tab < L.qt && L.qt < L.w && L.w < L.ut &&
        L.ut < L.ket && L.ket < L.p && L.p < L.gam);
  CHECK(a.grid_chunks >= 0 && a.grid_chunks <= L.max_chunks);
}

void fwd_cases() {
  // status strings
  CHECK(std::strcmp(kda_status_string(KDA_SUCCESS), "KDA_SUCCESS") == 0);
  CHECK(std::strcmp(kda_status_string(KDA_ERROR_LAUNCH_FAILED), "KDA_ERROR_LAUNCH_FAILED") == 0);
  CHECK(kda_version() > 0);

  // a valid call: both kernels, layout inside the workspace
  {
    reset();
    Fwd f;
    f.fit();
    CHECK(f.ws_bytes > 0);
    CHECK(f.run() == KDA_SUCCESS);
    CHECK(rec.intra == 1 && rec.inter == 1 && rec.epilogue == 0 && rec.check_cu == 0);
    CHECK(rec.fwd.grid_chunks == 2 * (2048 / 64));
    CHECK(rec.fwd.seq_len == 2048);
    layout_fits(rec.fwd, f.ws_bytes);
  }
  // every supported shape and both dtypes, varlen and equal lengths
  for (int dt = 0; dt < 2; ++dt)
    for (int d : {32, 64, 128})
      for (int C : {16, 32, 64})
        for (int varlen = 0; varlen < 2; ++varlen) {
          reset();
          Fwd f;
          f.dt = static_cast<kda_dtype>(dt);
          f.d = d;
          f.C = C;
          f.T = 1000;
          f.N = varlen ? 7 : 4;
          f.cu = varlen ? static_cast<const int32_t *>(dev(10)) : nullptr;
          f.fit();
          CHECK(f.ws_bytes > 0);
          CHECK(f.run() == KDA_SUCCESS);
          CHECK(rec.intra == 1 && rec.inter == 1);
          layout_fits(rec.fwd, f.ws_bytes);
          if (varlen) {
            CHECK(rec.fwd.grid_chunks == rec.fwd.lay.max_chunks);
            CHECK(rec.table == 1 && rec.table_entries == rec.fwd.lay.max_chunks);
            CHECK(reinterpret_cast<const char *>(rec.tab) ==
                  static_cast<const char *>(f.ws) + rec.fwd.lay.chunk_tab);
          } else {
            CHECK(rec.table == 0 && rec.fwd.chunk_tab == nullptr);
          }
        }
  // stages one at a time
  {
    Fwd f;
    f.fit();
    reset();
    f.stages = 1;
    CHECK(f.run() == KDA_SUCCESS && rec.intra == 1 && rec.inter == 0);
    reset();
    f.stages = 2;
    CHECK(f.run() == KDA_SUCCESS && rec.intra == 0 && rec.inter == 1);
    for (uint32_t bad : {0u, 4u, 7u}) {
      reset();
      f.stages = bad;
      CHECK(f.run() == KDA_ERROR_INVALID_VALUE && launches() == 0);
    }
  }
  // refusals before any launch
  auto refused = [](Fwd f, kda_status want, const char *what) {
    reset();
    const kda_status st = f.run();
    if (st != want || launches() != 0) {
      std::fprintf(stderr, "FAIL: %s: status %d, %d launches\n", what, (int)st, launches());
      ++failures;
    }
  };
  {
    Fwd f;
    f.fit();
    Fwd x = f;
    x.q = static_cast<const char *>(f.q) + 8;
    refused(x, KDA_ERROR_INVALID_VALUE, "misaligned q");
    x = f;
    x.beta = reinterpret_cast<const float *>(static_cast<const char *>(dev(5)) + 2);
    refused(x, KDA_ERROR_INVALID_VALUE, "misaligned beta");
    x = f;
    x.o = nullptr;
    refused(x, KDA_ERROR_INVALID_VALUE, "NULL o");
    x = f;
    x.ws = static_cast<char *>(f.ws) + 128;
    refused(x, KDA_ERROR_INVALID_VALUE, "workspace not 256-byte aligned");
    x = f;
    x.ws_bytes -= 1;
    refused(x, KDA_ERROR_INVALID_VALUE, "workspace one byte short");
    x = f;
    x.T = 4095;
    refused(x, KDA_ERROR_INVALID_VALUE, "T not a multiple of num_seqs without cu_seqlens");
    x = f;
    x.d = 96;
    refused(x, KDA_ERROR_NOT_SUPPORTED, "head size 96");
    x = f;
    x.C = 48;
    refused(x, KDA_ERROR_NOT_SUPPORTED, "chunk size 48");
    x = f;
    x.N = 0;
    refused(x, KDA_ERROR_INVALID_VALUE, "no sequences");
    x = f;
    x.T = -1;
    refused(x, KDA_ERROR_INVALID_VALUE, "negative token count");
    x = f;
    x.T = (int64_t)1 << 31;
    x.N = 1;
    refused(x, KDA_ERROR_NOT_SUPPORTED, "2^31 tokens");
    x = f;
    x.H = 70000;
    refused(x, KDA_ERROR_NOT_SUPPORTED, "70000 heads");
    x = f;
    x.s0 = reinterpret_cast<const float *>(static_cast<const char *>(dev(6)) + 4);
    refused(x, KDA_ERROR_INVALID_VALUE, "misaligned initial state");
    CHECK(kda_fwd_chunked_workspace_size(4096, 2, 8, 96, 96, 64, KDA_DTYPE_BF16) == 0);
    CHECK(kda_fwd_chunked_workspace_size(4096, 2, 8, 128, 64, 64, KDA_DTYPE_BF16) == 0);
    CHECK(kda_fwd_chunked_workspace_size((int64_t)1 << 40, 1, 8, 128, 128, 64,
                                         KDA_DTYPE_BF16) == 0);
  }
  // zero tokens: valid, nothing to read
  {
    reset();
    Fwd f;
    f.T = 0;
    f.q = f.k = f.v = f.g = f.o = nullptr;
    f.beta = nullptr;
    f.fit();
    CHECK(f.ws_bytes > 0);
    CHECK(f.run() == KDA_SUCCESS);
  }
  // options
  {
    Fwd f;
    f.fit();
    kda_options o{};
    f.opt = &o;
    reset();
    CHECK(f.run() == KDA_SUCCESS && rec.intra == 1 && rec.inter == 1);  // all-zero options
    // (enumerator values outside their enums, which C callers can pass, are
    // checked through ctypes in test_abi.py: in C++ merely forming them here
    // would be undefined behaviour in this driver)
    kda_options bad = o;
    f.opt = &bad;
    bad.gate = KDA_GATE_SOFTPLUS;
    refused(f, KDA_ERROR_INVALID_VALUE, "softplus gate without A");
    bad = o;
    bad.gate = KDA_GATE_SIGMOID;
    bad.gate_min = 0.f;
    refused(f, KDA_ERROR_INVALID_VALUE, "sigmoid gate with g_min = 0");
    bad.gate_min = std::nanf("");
    refused(f, KDA_ERROR_INVALID_VALUE, "sigmoid gate with NaN g_min");
    bad = o;
    bad.check_inputs = 1;
    refused(f, KDA_ERROR_INVALID_VALUE, "check_inputs without flags");
    bad = o;
    bad.out_gate = dev(11);
    refused(f, KDA_ERROR_INVALID_VALUE, "output gate without norm weight");
    bad = o;
    bad.out_norm_weight = static_cast<const float *>(dev(12));
    bad.out_norm_eps = std::nanf("");
    refused(f, KDA_ERROR_INVALID_VALUE, "NaN epsilon");
    bad = o;
    bad.state_slots = static_cast<const int32_t *>(dev(13));
    bad.num_slots = 0;
    refused(f, KDA_ERROR_INVALID_VALUE, "slots with an empty pool");
    // epilogue and checked cu_seqlens reach their launchers
    kda_options good = o;
    good.out_norm_weight = static_cast<const float *>(dev(12));
    good.out_norm_eps = 1e-6f;
    good.flags = static_cast<int32_t *>(dev(14));
    good.check_inputs = 1;
    Fwd g = f;
    g.opt = &good;
    g.cu = static_cast<const int32_t *>(dev(10));
    g.fit();
    reset();
    CHECK(g.run() == KDA_SUCCESS);
    CHECK(rec.check_cu == 1 && rec.intra == 1 && rec.inter == 1 && rec.epilogue == 1);
    CHECK(rec.epi_rows == g.T * g.H);
  }
  // a launch the runtime refuses
  {
    Fwd f;
    f.fit();
    reset();
    launch_result = hipErrorInvalidValue;
    CHECK(f.run() == KDA_ERROR_LAUNCH_FAILED);
    CHECK(rec.intra == 1 && rec.inter == 0);
  }
}

void decode_cases() {
  const void *q = dev(1), *k = dev(2), *v = dev(3);
  const float *g = static_cast<const float *>(dev(4)), *b = static_cast<const float *>(dev(5));
  float *st = static_cast<float *>(dev(6));
  void *o = dev(7);
  reset();
  CHECK(kda_decode_step(q, k, v, g, b, st, o, 256, 32, 128, 128, KDA_DTYPE_BF16, nullptr) ==
        KDA_SUCCESS);
  CHECK(rec.decode == 1 && rec.decode_batch == 256);
  reset();
  CHECK(kda_decode_step(q, k, v, g, b, st, o, 0, 32, 128, 128, KDA_DTYPE_BF16, nullptr) ==
        KDA_ERROR_INVALID_VALUE);
  CHECK(kda_decode_step(q, k, v, g, b, st, o, 4, 2, 96, 96, KDA_DTYPE_BF16, nullptr) ==
        KDA_ERROR_NOT_SUPPORTED);
  CHECK(kda_decode_step(q, k, v, g, b, static_cast<float *>(static_cast<void *>(
                                                static_cast<char *>(dev(6)) + 4)),
                        o, 4, 2, 128, 128, KDA_DTYPE_BF16, nullptr) == KDA_ERROR_INVALID_VALUE);
  CHECK(kda_decode_step(q, k, v, g, b, nullptr, o, 4, 2, 128, 128, KDA_DTYPE_BF16, nullptr) ==
        KDA_ERROR_INVALID_VALUE);
  CHECK(kda_decode_step(q, k, v, g, b, st, o, 1 << 30, 4, 128, 128, KDA_DTYPE_BF16, nullptr) ==
        KDA_ERROR_NOT_SUPPORTED);
  CHECK(launches() == 0);
  reset();
  launch_result = hipErrorInvalidValue;
  CHECK(kda_decode_step(q, k, v, g, b, st, o, 4, 2, 128, 128, KDA_DTYPE_F32, nullptr) ==
        KDA_ERROR_LAUNCH_FAILED);
}

void bwd_cases() {
  const int64_t T = 4096;
  const int32_t N = 2, H = 8, d = 128, C = 64;
  const size_t need = kda_bwd_chunked_workspace_size(T, N, H, d, d, C, KDA_DTYPE_BF16);
  CHECK(need > 0);
  auto call = [&](const void *q, size_t ws_bytes, int32_t dd) {
    return kda_bwd_chunked(q, dev(2), dev(3), static_cast<const float *>(dev(4)),
                           static_cast<const float *>(dev(5)), nullptr, N, T, H, dd, dd, C,
                           KDA_DTYPE_BF16, nullptr, dev(6), nullptr, dev(7), dev(8), dev(9),
                           static_cast<float *>(dev(10)), static_cast<float *>(dev(11)),
                           static_cast<float *>(dev(12)), dev(13), ws_bytes, nullptr);
  };
  reset();
  CHECK(call(dev(1), need, d) == KDA_SUCCESS && rec.bwd == 1);
  CHECK(rec.bwdargs.lay.total <= need);
  CHECK(rec.bwdargs.grid_chunks == 64);
  reset();
  CHECK(call(dev(1), need - 1, d) == KDA_ERROR_INVALID_VALUE && launches() == 0);
  CHECK(call(static_cast<const char *>(dev(1)) + 2, need, d) == KDA_ERROR_INVALID_VALUE);
  CHECK(call(dev(1), need, 96) == KDA_ERROR_NOT_SUPPORTED && launches() == 0);
}

}  // namespace

int main() {
  fwd_cases();
  decode_cases();
  bwd_cases();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi driver: all checks passed\n");
  return 0;
}
