// Validation paths of liblokafp8's C ABI, for a build whose api.cpp carries
// the address and undefined-behaviour sanitizers (tests/test_abi.py builds
// and runs it on the host).  Every pointer is an aligned placeholder that
// validation rejects or never reaches: no call here launches device work.
// With argument "nodevice" the HIP error path is checked as well (a host
// without a GPU).  Prints each mismatch; exits 1 if there is any.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../include/loka_fp8.h"

namespace {

int failures = 0;
void* const FAKE = reinterpret_cast<void*>(0x100000);
template <class T>
T* fk(size_t plus = 0) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(FAKE) + plus);
}

void expect(const char* what, long got, long want) {
  if (got != want) {
    std::printf("MISMATCH %s: got %ld, want %ld (%s)\n", what, got, want, loka_last_error());
    ++failures;
  }
}

loka_fwd_args fwd() {
  loka_fwd_args a;
  std::memset(&a, 0, sizeof a);
  a.M = 128; a.N = 256; a.K = 256; a.x_mode = LOKA_SCALE_ROW; a.eps = 1e-5f;
  a.x = FAKE; a.qw = fk<uint8_t>(); a.sw = FAKE; a.y = FAKE;
  return a;
}
loka_quant_args quant() {
  loka_quant_args a;
  std::memset(&a, 0, sizeof a);
  a.rows = 64; a.cols = 64; a.ld = 64; a.mode = LOKA_SCALE_ROW;
  a.src = FAKE; a.codes = fk<uint8_t>(); a.scales = FAKE;
  return a;
}
loka_bwd_args bwd() {
  loka_bwd_args a;
  std::memset(&a, 0, sizeof a);
  a.M = 128; a.N = 256; a.K = 256;
  a.dy = FAKE; a.qx = fk<uint8_t>(); a.sx = FAKE; a.mean = fk<float>(); a.rstd = fk<float>(); a.qw = fk<uint8_t>();
  a.sw = FAKE; a.x = FAKE; a.qw_row = fk<uint8_t>(); a.sw_row = fk<float>(); a.dx = FAKE; a.dw = fk<float>();
  return a;
}

void forward_cases() {
  loka_fwd_args a;
  a = fwd(); a.N = 100; expect("fwd N=100", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_UNSUPPORTED);
  a = fwd(); a.N = 0; expect("fwd N=0", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_UNSUPPORTED);
  a = fwd(); a.K = 20; expect("fwd K=20", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_UNSUPPORTED);
  a = fwd(); a.M = -1; expect("fwd M=-1", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); a.x_mode = 2; expect("fwd x_mode=2", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); a.x_mode = 9; expect("fwd x_mode=9", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); a.flags = 4; expect("fwd flags=4", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); a.eps = std::nanf(""); expect("fwd eps=nan", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); a.x = nullptr; expect("fwd x=null", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); a.x = fk<char>(8); expect("fwd x misaligned", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_ALIGNMENT);
  a = fwd(); a.z = fk<float>(4); expect("fwd z misaligned", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_ALIGNMENT);
  a = fwd(); a.x_mode = LOKA_SCALE_TENSOR; expect("fwd tensor ws", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_WORKSPACE);
  a = fwd(); expect("fwd row-major ws", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_WORKSPACE);
  a = fwd(); a.flags = 2; a.gamma = FAKE; expect("fwd blocknorm gamma", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); expect("fwd ws row-major", (long)loka_gemm_fp8_ln_workspace_size(&a), 256 * 256);
  a = fwd(); a.flags = LOKA_FWD_W_PACKED; expect("fwd ws packed", (long)loka_gemm_fp8_ln_workspace_size(&a), 0);
  a = fwd(); a.M = 0; a.x = nullptr; a.qw = nullptr; a.sw = nullptr; a.y = nullptr;
  expect("fwd empty", loka_gemm_fp8_ln(&a, nullptr), LOKA_OK);
  a = fwd(); a.M = -1; expect("noalloc M=-1", loka_gemm_fp8_ln_noalloc(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = fwd(); a.M = 0; a.x = nullptr; a.qw = nullptr; a.sw = nullptr; a.y = nullptr;
  expect("noalloc empty", loka_gemm_fp8_ln_noalloc(&a, nullptr), LOKA_OK);
}

void quant_cases() {
  loka_quant_args a;
  a = quant(); a.rows = -1; expect("quant rows=-1", loka_quant_fp8(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = quant(); a.ld = 32; expect("quant ld=32", loka_quant_fp8(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = quant(); a.fmt = 3; expect("quant fmt=3", loka_quant_fp8(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = quant(); a.transpose_out = 4; expect("quant trans=4", loka_quant_fp8(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = quant(); a.transpose_out = 3; a.rows = 40;
  expect("quant trans=3 rows=40", loka_quant_fp8(&a, nullptr), LOKA_ERR_UNSUPPORTED);
  a = quant(); a.codes = fk<uint8_t>(1); expect("quant codes misaligned", loka_quant_fp8(&a, nullptr), LOKA_ERR_ALIGNMENT);
  a = quant(); a.mode = LOKA_SCALE_TENSOR; expect("quant tensor ws", loka_quant_fp8(&a, nullptr), LOKA_ERR_WORKSPACE);
  a = quant(); a.rows = 0; a.src = nullptr; a.codes = nullptr; a.scales = nullptr;
  expect("quant empty", loka_quant_fp8(&a, nullptr), LOKA_OK);
  a = quant(); a.mode = LOKA_SCALE_MX32_ROW; expect("quant mx ws", (long)loka_quant_workspace_size(&a), 0);
}

void backward_cases() {
  loka_bwd_args a;
  a = bwd(); a.flags = 16; expect("bwd flags=16", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = bwd(); a.K = 96; expect("bwd K=96", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_UNSUPPORTED);
  a = bwd(); a.flags = LOKA_BWD_MX32_SQ | LOKA_BWD_W_PACKED; a.qw_row = nullptr;
  expect("bwd sq+packed without qw_row", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = bwd(); a.flags = LOKA_BWD_MX32_SQ; a.xc_codes = fk<uint8_t>();
  expect("bwd sq+col outputs", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = bwd(); a.dz = fk<float>(4); expect("bwd dz misaligned", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_ALIGNMENT);
  a = bwd(); a.dw = nullptr; expect("bwd dw=null", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = bwd(); a.flags = LOKA_BWD_NO_LN; a.dgamma = fk<float>();
  expect("bwd no_ln dgamma", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_INVALID_ARG);
  a = bwd(); expect("bwd ws", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_WORKSPACE);
  a = bwd(); a.flags = LOKA_BWD_W_PACKED; expect("bwd packed ws", loka_gemm_fp8_bwd(&a, nullptr), LOKA_ERR_WORKSPACE);
  a = bwd(); a.M = 16384; a.N = 512; a.K = 512;
  const size_t row = loka_gemm_fp8_bwd_workspace_size(&a);
  a.flags = LOKA_BWD_MX32_SQ;
  const size_t sq = loka_gemm_fp8_bwd_workspace_size(&a);
  expect("bwd ws square smaller", (long)(row >= sq + 16384ull * 512 * 4), 1);
}

void other_cases() {
  loka_group_desc d[2];
  std::memset(d, 0, sizeof d);
  for (auto& g : d) {
    g.M = 64; g.N = 128; g.K = 128; g.x = FAKE; g.qw = fk<uint8_t>(); g.sw = fk<float>(); g.y = FAKE;
  }
  d[1].N = 96;
  loka_grouped_args ga;
  std::memset(&ga, 0, sizeof ga);
  ga.num_groups = 2; ga.x_mode = LOKA_SCALE_ROW; ga.eps = 1e-5f; ga.groups = d;
  expect("grouped N=96", loka_grouped_gemm_fp8_ln(&ga, nullptr), LOKA_ERR_UNSUPPORTED);
  d[1].N = 128; d[1].y = fk<char>(2);
  expect("grouped y misaligned", loka_grouped_gemm_fp8_ln(&ga, nullptr), LOKA_ERR_ALIGNMENT);
  d[1].y = FAKE;
  expect("grouped ws", loka_grouped_gemm_fp8_ln(&ga, nullptr), LOKA_ERR_WORKSPACE);
  ga.num_groups = 0;
  expect("grouped empty", loka_grouped_gemm_fp8_ln(&ga, nullptr), LOKA_OK);

  loka_probe_input_args pi;
  std::memset(&pi, 0, sizeof pi);
  pi.B = 16; pi.K = 0; pi.T = FAKE; pi.mu = fk<float>(); pi.S = fk<float>();
  expect("probe K=0", loka_probe_input_update(&pi, nullptr), LOKA_ERR_UNSUPPORTED);
  pi.K = 64;
  expect("probe ws", loka_probe_input_update(&pi, nullptr), LOKA_ERR_WORKSPACE);
  loka_probe_weight_args pw;
  std::memset(&pw, 0, sizeof pw);
  pw.R = 64; pw.C = 64; pw.m = 1.0f; pw.W = FAKE; pw.M = fk<float>(); pw.U = fk<float>(); pw.V = fk<float>();
  pw.info = fk<int32_t>();
  expect("probe m=1", loka_probe_weight_update(&pw, nullptr), LOKA_ERR_INVALID_ARG);
  loka_mere_args ma;
  std::memset(&ma, 0, sizeof ma);
  ma.M = 64; ma.N = 64; ma.K = 4096; ma.S = 8; ma.x = FAKE; ma.w = FAKE; ma.z = fk<float>();
  ma.rows = fk<int64_t>(); ma.out = fk<double>();
  expect("mere K=4096", loka_mere_z(&ma, nullptr), LOKA_ERR_UNSUPPORTED);
  ma.K = 64;
  expect("mere ws size", (long)loka_mere_workspace_size(&ma), 8 * 3 * 8);

  loka_dispatch_candidate c[3] = {{10.0, 0.1}, {8.0, 0.3}, {9.0, 0.15}};
  int32_t choice = -2;
  expect("dispatch status", loka_dispatch_select(c, 3, 12.0, 0.2, 1.05, &choice), LOKA_OK);
  expect("dispatch choice", choice, 2);
  expect("dispatch null", loka_dispatch_select(nullptr, 3, 12.0, 0.2, 1.05, &choice), LOKA_ERR_INVALID_ARG);
  for (int s = 0; s <= 5; ++s) expect("status string", loka_status_string((loka_status)s) != nullptr, 1);
  expect("status string unknown", loka_status_string((loka_status)99) != nullptr, 1);
  expect("abi", loka_abi_version(), LOKA_ABI_VERSION);
}

}  // namespace

int main(int argc, char** argv) {
  forward_cases();
  quant_cases();
  backward_cases();
  other_cases();
  if (argc > 1 && std::strcmp(argv[1], "nodevice") == 0) {
    loka_fwd_args a = fwd();
    a.flags = LOKA_FWD_W_PACKED;
    expect("fwd without a device", loka_gemm_fp8_ln(&a, nullptr), LOKA_ERR_HIP);
    expect("error names the call", std::strstr(loka_last_error(), "loka_gemm_fp8_ln") != nullptr, 1);
  }
  std::printf("%d mismatch(es)\n", failures);
  return failures == 0 ? 0 : 1;
}
