// Host-only checks of the C ABI's validation and argument marshalling
// (gdn_api.cpp linked against the launcher stand-ins of launch_stubs.cpp),
// built with the address and undefined-behaviour sanitizers: every status
// code of include/gdn.h is reached, every valid call hands its launcher the
// sizes and pointers it was given, and no call reads or writes memory it
// does not own on the host.  Prints one line per failed check and a summary.
#include <cstdio>
#include <cstring>

#include "../../include/gdn.h"
#include "launch_stubs.hpp"

static int n_checks = 0, n_failed = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    ++n_checks;                                                         \
    if (!(cond)) {                                                      \
      ++n_failed;                                                       \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);             \
    }                                                                   \
  } while (0)

// A fake device buffer: aligned host memory never dereferenced by the API.
alignas(256) static unsigned char arena[1 << 16];
static void* P(int k) { return arena + 256 * k; }
static const int32_t* I(int k) { return reinterpret_cast<const int32_t*>(P(k)); }
static float* F(int k) { return reinterpret_cast<float*>(P(k)); }
static const uint8_t* U(int k) { return reinterpret_cast<const uint8_t*>(P(k)); }
static void* MIS(int k) { return arena + 256 * k + 2; }  // 2-byte aligned only

static bool launched(const char* fn) { return stub::last.which && std::strcmp(stub::last.which, fn) == 0; }
static void reset() { stub::last = stub::Record{}; stub::next_result = hipSuccess; }

static const gdn_dims QWEN{16, 32, 128, 128, 4};

static void dims_checks() {
  gdn_dims d = QWEN;
  const int64_t T = 100;
  auto fwd = [&](const gdn_dims* dd) {
    return gdn_conv1d_fwd(dd, GDN_BF16, 1, T, P(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6), nullptr);
  };
  CHECK(fwd(nullptr) == GDN_ERR_NULL);
  for (int f = 0; f < 5; ++f) {   // each field zero, then negative
    d = QWEN;
    int32_t* fld[] = {&d.h_k, &d.h_v, &d.d_k, &d.d_v, &d.conv_w};
    *fld[f] = 0;
    CHECK(fwd(&d) == GDN_ERR_SHAPE);
    *fld[f] = -3;
    CHECK(fwd(&d) == GDN_ERR_SHAPE);
  }
  d = QWEN; d.h_v = 24;                              // not a multiple of h_k
  CHECK(fwd(&d) == GDN_ERR_SHAPE);
  d = QWEN; d.d_v = 64;                              // d_k != d_v
  CHECK(fwd(&d) == GDN_ERR_UNSUPPORTED);
  d = QWEN; d.d_k = d.d_v = 96;
  CHECK(fwd(&d) == GDN_ERR_UNSUPPORTED);
  d = QWEN; d.conv_w = 5;
  CHECK(fwd(&d) == GDN_ERR_UNSUPPORTED);
  d = QWEN; d.h_k = 1 << 20; d.h_v = 1 << 20;        // c_ch beyond 2^24
  CHECK(fwd(&d) == GDN_ERR_UNSUPPORTED);
  d = QWEN; d.h_k = 0x7fffffff; d.h_v = 0x7fffffff;  // the size check must not overflow
  CHECK(fwd(&d) == GDN_ERR_UNSUPPORTED);
  reset();
  CHECK(fwd(&QWEN) == GDN_OK && launched("launch_conv1d_fwd"));
}

static void conv_checks() {
  reset();
  CHECK(gdn_conv1d_fwd(&QWEN, 7, 1, 10, P(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6), nullptr) ==
        GDN_ERR_DTYPE);
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, -1, 10, P(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6), nullptr) ==
        GDN_ERR_SHAPE);
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 0, 10, P(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6), nullptr) ==
        GDN_ERR_SHAPE);
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 8,
                       nullptr, nullptr) == GDN_OK && !stub::last.which);
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 2, 10, nullptr, P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6),
                       nullptr) == GDN_ERR_NULL);
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 2, 10, P(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(1),
                       nullptr) == GDN_ERR_SHAPE);     // y aliases x
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 2, 10, MIS(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6),
                       nullptr) == GDN_ERR_ALIGN);
  // two empty sequences: no x or y needed
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 2, 0, nullptr, P(2), nullptr, I(3), I(4), nullptr, P(5), 8, nullptr,
                       nullptr) == GDN_OK && launched("launch_conv1d_fwd"));
  reset();
  const int64_t big = (int64_t)3 << 32;               // offsets past 2^32 tokens stay 64-bit
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_F32, 5, big, P(1), P(2), P(7), I(3), I(4), U(8), P(5), 9, P(6), nullptr) ==
        GDN_OK);
  CHECK(launched("launch_conv1d_fwd") && stub::last.conv_fwd.t_total == big && stub::last.conv_fwd.n_seq == 5 &&
        !stub::last.conv_fwd.bf16 && stub::last.conv_fwd.n_slots == 9 && stub::last.conv_fwd.bias == P(7) &&
        stub::last.conv_fwd.has_init == U(8) && stub::last.conv_fwd.y == P(6) &&
        stub::last.conv_fwd.s.c_ch() == 2 * 16 * 128 + 32 * 128);
  stub::next_result = hipErrorInvalidValue;          // a failed launch maps to GDN_ERR_HIP
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 1, 10, P(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6), nullptr) ==
        GDN_ERR_HIP);
  reset();
  CHECK(gdn_conv1d_update(&QWEN, GDN_BF16, 4, -1, P(1), P(2), nullptr, P(3), 8, I(4), nullptr, P(5), nullptr) ==
        GDN_ERR_SHAPE);
  CHECK(gdn_conv1d_update(&QWEN, GDN_BF16, 4, 0, nullptr, nullptr, nullptr, nullptr, 8, nullptr, nullptr, nullptr,
                          nullptr) == GDN_OK && !stub::last.which);
  CHECK(gdn_conv1d_update(&QWEN, GDN_BF16, 4, 2, P(1), P(2), nullptr, P(3), 8, nullptr, nullptr, P(5), nullptr) ==
        GDN_ERR_NULL);
  CHECK(gdn_conv1d_update(&QWEN, GDN_BF16, 4, 2, P(1), P(2), nullptr, MIS(3), 8, I(4), nullptr, P(5), nullptr) ==
        GDN_ERR_ALIGN);
  CHECK(gdn_conv1d_update(&QWEN, GDN_BF16, 4, 2, P(1), P(2), nullptr, P(3), 8, I(4), I(6), P(5), nullptr) ==
        GDN_OK);
  CHECK(launched("launch_conv1d_update") && stub::last.conv_update.t_step == 2 &&
        stub::last.conv_update.out_slots == I(6) && stub::last.conv_update.n_slots == 8);
}

static void gating_checks() {
  reset();
  CHECK(gdn_gating(GDN_BF16, 10, 0, P(1), P(2), F(3), F(4), F(5), F(6), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_gating(GDN_BF16, -1, 32, P(1), P(2), F(3), F(4), F(5), F(6), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_gating(GDN_BF16, 10, 32, P(1), P(2), F(3), nullptr, F(5), F(6), nullptr) == GDN_ERR_NULL);
  CHECK(gdn_gating(GDN_BF16, 0, 32, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == GDN_OK &&
        !stub::last.which);
  CHECK(gdn_gating(GDN_F32, 10, 32, P(1), P(2), F(3), F(4), F(5), F(6), nullptr) == GDN_OK);
  CHECK(launched("launch_gating") && stub::last.gating.n_tokens == 10 && stub::last.gating.h_v == 32 &&
        stub::last.gating.beta == F(6) && !stub::last.gating.bf16);
}

static void prefill_checks() {
  const int64_t T = 4096;
  const size_t ws = gdn_prefill_workspace_size(&QWEN, GDN_BF16, 2, T, 64);
  CHECK(ws > 0 && ws == gdn_chunk_prefill_workspace_size(&QWEN, GDN_BF16, 2, T, 64));
  CHECK(gdn_prefill_workspace_size(nullptr, GDN_BF16, 2, T, 64) == 0);
  CHECK(gdn_prefill_workspace_size(&QWEN, 9, 2, T, 64) == 0);
  CHECK(gdn_prefill_workspace_size(&QWEN, GDN_BF16, -2, T, 64) == 0);
  // row counts past 2^40 are refused, so no workspace size can wrap
  const int64_t huge = (int64_t)1 << 62;
  CHECK(gdn_prefill_workspace_size(&QWEN, GDN_BF16, 2, huge, 64) == 0);
  CHECK(gdn_chunk_prefill_workspace_size(&QWEN, GDN_BF16, 2, huge, 64) == 0);
  CHECK(gdn_prefill_workspace_size(&QWEN, GDN_BF16, 2, (int64_t)1 << 40, 64) > 0);
  CHECK(gdn_chunk_prefill(&QWEN, GDN_BF16, 2, huge, 64, 1.0f, P(1), F(2), F(3), I(4), I(5), U(6), F(7), 8, P(8),
                          nullptr, nullptr, 1e-6f, P(20), 64, nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_prefill(&QWEN, GDN_BF16, 2, huge, 64, 1.0f, P(1), P(2), nullptr, P(3), P(4), F(5), F(6), I(7), I(8),
                    U(9), P(14), F(10), 8, P(11), nullptr, nullptr, 1e-6f, P(20), 64, nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_conv1d_fwd(&QWEN, GDN_BF16, 2, huge, P(1), P(2), nullptr, I(3), I(4), nullptr, P(5), 8, P(6),
                       nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_gating(GDN_BF16, huge, 32, P(1), P(2), F(3), F(4), F(5), F(6), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_rmsnorm_gemma(GDN_BF16, huge, 2048, P(1), P(2), 1e-6f, P(3), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_in_proj(&QWEN, GDN_BF16, huge, 2048, P(1), P(2), P(3), P(4), P(5), P(6), P(7), nullptr) ==
        GDN_ERR_SHAPE);
  CHECK(gdn_out_proj(&QWEN, GDN_BF16, huge, 2048, P(1), P(2), nullptr, P(4), nullptr) == GDN_ERR_SHAPE);
  auto chunk = [&](int32_t n, int64_t t, int32_t c, const void* qkv, const void* z, const void* nw, float eps,
                   void* w, size_t wb) {
    return gdn_chunk_prefill(&QWEN, GDN_BF16, n, t, c, 1.0f, qkv, F(2), F(3), I(4), I(5), U(6), F(7), 8, P(8), z,
                             nw, eps, w, wb, nullptr);
  };
  reset();
  CHECK(chunk(2, T, 48, P(1), nullptr, nullptr, 1e-6f, P(20), ws) == GDN_ERR_UNSUPPORTED);
  CHECK(chunk(0, T, 64, P(1), nullptr, nullptr, 1e-6f, P(20), ws) == GDN_ERR_SHAPE);
  CHECK(chunk(2, T, 64, nullptr, nullptr, nullptr, 1e-6f, P(20), ws) == GDN_ERR_NULL);
  CHECK(chunk(2, T, 64, P(1), P(9), nullptr, 1e-6f, P(20), ws) == GDN_ERR_NULL);   // z without norm_w
  CHECK(chunk(2, T, 64, P(1), P(9), P(10), -1.0f, P(20), ws) == GDN_ERR_SHAPE);
  float nan;
  const unsigned bits = 0x7fc00000u;
  std::memcpy(&nan, &bits, 4);
  CHECK(chunk(2, T, 64, P(1), P(9), P(10), nan, P(20), ws) == GDN_ERR_SHAPE);
  CHECK(chunk(2, T, 64, P(1), MIS(9), P(10), 1e-6f, P(20), ws) == GDN_ERR_ALIGN);
  CHECK(chunk(2, T, 64, P(1), P(9), P(10), 1e-6f, nullptr, ws) == GDN_ERR_WORKSPACE);
  CHECK(chunk(2, T, 64, P(1), P(9), P(10), 1e-6f, P(20), ws - 1) == GDN_ERR_WORKSPACE);
  CHECK(!stub::last.which);
  CHECK(chunk(2, T, 64, P(1), P(9), P(10), 1e-6f, P(20), ws) == GDN_OK);
  CHECK(launched("launch_chunk_split") && stub::last.chunk.t_total == T && stub::last.chunk.chunk == 64 &&
        stub::last.chunk.ws_bytes == ws && stub::last.chunk.z == P(9) && stub::last.chunk.x == nullptr);

  auto fused = [&](const void* x, const void* conv_state, void* w, size_t wb) {
    return gdn_prefill(&QWEN, GDN_BF16, 2, T, 64, 0.5f, x, P(2), nullptr, P(3), P(4), F(5), F(6), I(7), I(8),
                       U(9), const_cast<void*>(conv_state), F(10), 8, P(11), P(12), P(13), 1e-6f, w, wb, nullptr);
  };
  reset();
  CHECK(fused(P(1), nullptr, P(20), ws) == GDN_ERR_NULL);
  CHECK(fused(MIS(1), P(14), P(20), ws) == GDN_ERR_ALIGN);
  CHECK(fused(P(1), P(14), P(20), ws / 2) == GDN_ERR_WORKSPACE);
  CHECK(fused(P(1), P(14), P(20), ws) == GDN_OK);
  CHECK(launched("launch_prefill_fused") && stub::last.chunk.x == P(1) && stub::last.chunk.conv_state == P(14) &&
        stub::last.chunk.a_in == P(3) && stub::last.chunk.b_in == P(4) && stub::last.chunk.A_log == F(5) &&
        stub::last.chunk.dt_bias == F(6) && stub::last.chunk.scale == 0.5f && stub::last.chunk.o == P(11));
}

static void decode_checks() {
  reset();
  auto rec = [&](int32_t n, int32_t t, const void* z, const void* nw, void* o) {
    return gdn_recurrent_decode(&QWEN, GDN_BF16, n, t, 1.0f, P(1), P(2), P(3), F(4), F(5), F(6), 64, I(7), I(8), o,
                                z, nw, 1e-6f, nullptr);
  };
  CHECK(rec(-1, 1, nullptr, nullptr, P(9)) == GDN_ERR_SHAPE);
  CHECK(rec(4, 0, nullptr, nullptr, nullptr) == GDN_OK && !stub::last.which);
  CHECK(rec(4, 1, nullptr, nullptr, nullptr) == GDN_ERR_NULL);
  CHECK(rec(4, 1, P(10), nullptr, P(9)) == GDN_ERR_NULL);
  CHECK(rec(4, 1, MIS(10), P(11), P(9)) == GDN_ERR_ALIGN);
  CHECK(rec(4, 3, P(10), P(11), P(9)) == GDN_OK && launched("launch_recurrent") &&
        stub::last.recurrent.t_step == 3 && stub::last.recurrent.out_slots == I(8));
  reset();
  gdn_dims d3 = QWEN;
  d3.h_v = 48;                                         // h_v = 3 h_k: not a decode shape
  CHECK(gdn_decode(&d3, GDN_BF16, 4, 1, 1.0f, P(1), P(2), nullptr, P(3), P(4), F(5), F(6), P(7), F(8), 64, I(9),
                   nullptr, P(10), nullptr, nullptr, 1e-6f, nullptr) == GDN_ERR_UNSUPPORTED);
  CHECK(gdn_decode(&QWEN, GDN_BF16, 4, 1, 1.0f, P(1), P(2), nullptr, P(3), P(4), F(5), F(6), nullptr, F(8), 64, I(9),
                   nullptr, P(10), nullptr, nullptr, 1e-6f, nullptr) == GDN_ERR_NULL);
  CHECK(gdn_decode(&QWEN, GDN_BF16, 4, 2, 1.0f, P(1), P(2), P(12), P(3), P(4), F(5), F(6), P(7), F(8), 64, I(9),
                   I(11), P(10), P(13), P(14), 1e-6f, nullptr) == GDN_OK);
  CHECK(launched("launch_decode") && stub::last.decode.conv_b == P(12) && stub::last.decode.out_slots == I(11) &&
        stub::last.decode.z == P(13) && stub::last.decode.n_slots == 64);
  reset();
  CHECK(gdn_state_copy(&QWEN, GDN_BF16, F(1), nullptr, 8, I(2), I(3), -1, nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_state_copy(&QWEN, GDN_BF16, F(1), nullptr, 8, nullptr, I(3), 2, nullptr) == GDN_ERR_NULL);
  CHECK(gdn_state_copy(&QWEN, GDN_BF16, F(1), MIS(4), 8, I(2), I(3), 2, nullptr) == GDN_ERR_ALIGN);
  CHECK(gdn_state_copy(&QWEN, GDN_BF16, F(1), P(4), 8, I(2), I(3), 2, nullptr) == GDN_OK &&
        launched("launch_state_copy") && stub::last.state_copy.n == 2 && stub::last.state_copy.conv_state == P(4));
}

static void block_checks() {
  reset();
  CHECK(gdn_rmsnorm_gemma(GDN_BF16, 4, 12, P(1), P(2), 1e-6f, P(3), nullptr) == GDN_ERR_SHAPE);   // hidden % 8
  CHECK(gdn_rmsnorm_gemma(GDN_BF16, 4, 2048, P(1), P(2), -1.0f, P(3), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_rmsnorm_gemma(GDN_BF16, 4, 2048, P(1), nullptr, 1e-6f, P(3), nullptr) == GDN_ERR_NULL);
  CHECK(gdn_rmsnorm_gemma(GDN_BF16, 4, 2048, P(1), P(2), 1e-6f, MIS(3), nullptr) == GDN_ERR_ALIGN);
  CHECK(gdn_rmsnorm_gemma(GDN_BF16, 4, 2048, P(1), P(2), 1e-6f, P(3), nullptr) == GDN_OK &&
        launched("launch_gemma_norm") && stub::last.norm.rows == 4 && stub::last.norm.hidden == 2048);
  reset();
  CHECK(gdn_in_proj(&QWEN, GDN_F32, 4, 2048, P(1), P(2), P(3), P(4), P(5), P(6), P(7), nullptr) ==
        GDN_ERR_UNSUPPORTED);
  CHECK(gdn_in_proj(&QWEN, GDN_BF16, 4, 2047, P(1), P(2), P(3), P(4), P(5), P(6), P(7), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_in_proj(&QWEN, GDN_BF16, 4, 2048, P(1), P(2), P(3), P(4), nullptr, P(6), P(7), nullptr) ==
        GDN_ERR_NULL);
  CHECK(gdn_in_proj(&QWEN, GDN_BF16, 4, 2048, P(1), P(2), P(3), P(4), P(5), P(6), P(7), nullptr) == GDN_OK);
  const gdn::ProjArgs& p = stub::last.proj;
  const int c_ch = 2 * 16 * 128 + 32 * 128, vd = 32 * 128;
  CHECK(launched("launch_proj") && p.m == 4 && p.k == 2048 && p.nseg == 4 && p.n == c_ch + vd + 64 &&
        p.n_w0 == c_ch + vd && p.w1 == P(3) && p.residual == nullptr);
  // the segments tile [0, n) in order: qkv | z | b | a
  CHECK(p.seg[0].begin == 0 && p.seg[1].begin == c_ch && p.seg[2].begin == c_ch + vd &&
        p.seg[3].begin == c_ch + vd + 32 && p.seg[3].begin + p.seg[3].ld == p.n);
  CHECK(p.seg[0].ptr == P(4) && p.seg[1].ptr == P(5) && p.seg[2].ptr == P(6) && p.seg[3].ptr == P(7));
  CHECK(p.seg[0].ld == c_ch && p.seg[1].ld == vd && p.seg[2].ld == 32 && p.seg[3].ld == 32);
  reset();
  CHECK(gdn_out_proj(&QWEN, GDN_BF16, 4, 2048, P(1), P(2), MIS(3), P(4), nullptr) == GDN_ERR_ALIGN);
  CHECK(gdn_out_proj(&QWEN, GDN_BF16, 0, 2048, nullptr, nullptr, nullptr, nullptr, nullptr) == GDN_OK &&
        !stub::last.which);
  CHECK(gdn_out_proj(&QWEN, GDN_BF16, 4, 2048, P(1), P(2), P(3), P(4), nullptr) == GDN_OK);
  CHECK(launched("launch_proj") && stub::last.proj.nseg == 1 && stub::last.proj.k == vd &&
        stub::last.proj.n == 2048 && stub::last.proj.residual == P(3) && stub::last.proj.ld_res == 2048);
}

static void slot_checks() {
  reset();
  CHECK(gdn_check_slots(-1, I(1), 4, nullptr, 0, reinterpret_cast<int32_t*>(P(2)), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_check_slots(8, I(1), -4, nullptr, 0, reinterpret_cast<int32_t*>(P(2)), nullptr) == GDN_ERR_SHAPE);
  CHECK(gdn_check_slots(8, I(1), 4, nullptr, 3, reinterpret_cast<int32_t*>(P(2)), nullptr) == GDN_ERR_NULL);
  CHECK(gdn_check_slots(8, I(1), 4, nullptr, 0, nullptr, nullptr) == GDN_ERR_NULL);
  CHECK(gdn_check_slots(8, nullptr, 0, nullptr, 0, nullptr, nullptr) == GDN_OK && !stub::last.which);
  CHECK(gdn_check_slots(8, I(1), 4, I(3), 12, reinterpret_cast<int32_t*>(P(2)), nullptr) == GDN_OK);
  CHECK(launched("launch_slot_check") && stub::last.slot_check.n == 4 && stub::last.slot_check.n_out == 12 &&
        stub::last.slot_check.out_slots == I(3) && stub::last.slot_check.n_slots == 8);
}

static void status_checks() {
  const int codes[] = {GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE,
                       GDN_ERR_HIP, GDN_ERR_ALIGN, GDN_ERR_TOO_LARGE, 12345, -999};
  for (int c : codes) {
    const char* s = gdn_status_string(c);
    CHECK(s != nullptr && std::strlen(s) > 0);
  }
  CHECK(std::strcmp(gdn_status_string(GDN_OK), "GDN_OK") == 0);
  CHECK(gdn_version() != nullptr);
}

int main() {
  dims_checks();
  conv_checks();
  gating_checks();
  prefill_checks();
  decode_checks();
  block_checks();
  slot_checks();
  status_checks();
  std::printf("host API checks: %d run, %d failed\n", n_checks, n_failed);
  return n_failed ? 1 : 0;
}
