// attn_self_test: a tiny selection and attention run on the current device,
// checked against values that follow from how its inputs are built, for a
// start-up check that fails fast and names the library, its version and the
// GPU (the tiny plan-and-run check of mstar PR #927, "Since the review").
//
// The inputs make every expected value exact:
// - the 128 real keys are scaled one-hot vectors, 16 * e_r for key rank r
//   (prefix keys first, then generation keys), so with softmax scale 1 a
//   query 16 * e_t has logit 256 on the key of rank t and 0 on every other
//   key: e^-256 underflows in fp32, so a row whose target key is visible
//   returns that key's value row exactly, and a row whose target is not
//   visible weights every visible key equally (their mean, rounded once);
// - values are multiples of 1/16 below 2 in magnitude (exact in bf16);
// - padded query rows and padded keys and values hold NaN, which must not
//   reach any output.
// The selector's choice among candidate blocks is not predicted: its list is
// checked for structure (count, order, range, protected block first), and
// the attention output is checked against the closed form for that list.
//
// This is a start-up check, not a call path: it allocates its own device
// buffers, runs on the null stream and synchronises the device.

#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "bsattn.h"
#include "internal.h"

namespace {

constexpr int kD = 128, kHq = 2, kHkv = 1, kBlock = 64;
constexpr int kQLen = 128, kQValid = 100;
constexpr int kPrefixLen = 64, kPrefixValid = 40;
constexpr int kKvLen = 192, kSuffixValid = 88;  // 40 + 88 = 128 real keys
constexpr int kNk = kKvLen / kBlock, kNq = kQLen / kBlock;
constexpr int kRowStride = kNk;                 // one slot more than the kept blocks
constexpr uint16_t kNaN = 0x7FC0;

uint16_t bf16_of(float x) {  // exact for the values used here
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

float float_of(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

// Sequence position of the key of rank r, and the rank of a position (-1 for padding).
int pos_of_rank(int r) { return r < kPrefixValid ? r : kPrefixLen + (r - kPrefixValid); }
int rank_of_pos(int p) {
  if (p < kPrefixLen) return p < kPrefixValid ? p : -1;
  return p - kPrefixLen < kSuffixValid ? kPrefixValid + (p - kPrefixLen) : -1;
}
int target_rank(int t, int h) { return (t * 37 + 11 * h) % (kPrefixValid + kSuffixValid); }
float value_at(int p, int d) { return (float)((p * 131 + d * 17) % 61 - 30) / 16.0f; }

struct DeviceBuffers {
  void* base = nullptr;
  ~DeviceBuffers() {
    if (base != nullptr) (void)hipFree(base);
  }
};

struct Checker {
  char msg[384] = {0};
  bool failed = false;
  void fail_at(const char* what, int h, int t, int d, double got, double want) {
    if (failed) return;
    failed = true;
    snprintf(msg, sizeof msg, "%s: head %d row %d dim %d: got %.9g, expected %.9g", what, h, t, d,
             got, want);
  }
  void fail_msg(const char* text) {
    if (failed) return;
    failed = true;
    snprintf(msg, sizeof msg, "%s", text);
  }
};

// Output of row (h, t) over the visible key ranks [vis(r) true]: the target
// key's value row if it is visible, else the mean of the visible value rows.
template <class Visible>
void expect_row(Checker& c, const char* what, const std::vector<uint16_t>& out, int h, int t,
                Visible vis) {
  const int tr = target_rank(t, h);
  const uint16_t* o = out.data() + ((size_t)t * kHq + h) * kD;
  if (vis(tr)) {
    const int p = pos_of_rank(tr);
    for (int d = 0; d < kD; ++d)
      if (o[d] != bf16_of(value_at(p, d))) c.fail_at(what, h, t, d, float_of(o[d]), value_at(p, d));
    return;
  }
  int n = 0;
  std::vector<double> sum(kD, 0.0);
  for (int r = 0; r < kPrefixValid + kSuffixValid; ++r)
    if (vis(r)) {
      ++n;
      for (int d = 0; d < kD; ++d) sum[d] += value_at(pos_of_rank(r), d);
    }
  for (int d = 0; d < kD; ++d) {
    const double want = n > 0 ? sum[d] / n : 0.0;
    const double got = float_of(o[d]);
    // one fp32 division and one bf16 rounding away from the exact mean
    if (!(std::fabs(got - want) <= std::fabs(want) * (1.0 / 128) + 1e-6))
      c.fail_at(what, h, t, d, got, want);
  }
}

void expect_padded_rows_zero(Checker& c, const char* what, const std::vector<uint16_t>& out) {
  for (int t = kQValid; t < kQLen; ++t)
    for (int h = 0; h < kHq; ++h)
      for (int d = 0; d < kD; ++d) {
        const uint16_t x = out[((size_t)t * kHq + h) * kD + d];
        if (x != 0 && x != 0x8000) c.fail_at(what, h, t, d, float_of(x), 0.0);
      }
}

}  // namespace

extern "C" attn_status attn_self_test(void) {
  const char* fn = "attn_self_test";
  int dev = -1;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return bsattn::report(ATTN_ERR_DEVICE, fn, "no HIP device available");
  char where[160];
  snprintf(where, sizeof where, "device %d (%s)", dev, prop.gcnArchName);

  attn_shape s{};
  s.batch = 1;
  s.num_q_heads = kHq;
  s.num_kv_heads = kHkv;
  s.head_dim = kD;
  s.block_q = kBlock;
  s.block_k = kBlock;
  s.q_len = kQLen;
  s.q_valid = kQValid;
  s.kv_prefix_len = kPrefixLen;
  s.kv_prefix_valid = kPrefixValid;
  s.kv_len = kKvLen;
  s.kv_suffix_valid = kSuffixValid;
  const int64_t qst[3] = {(int64_t)kQLen * kHq * kD, kHq * kD, kD};
  const int64_t kst[3] = {(int64_t)kKvLen * kHkv * kD, kHkv * kD, kD};
  for (int i = 0; i < 3; ++i) {
    s.q_stride[i] = qst[i];
    s.o_stride[i] = qst[i];
    s.k_stride[i] = kst[i];
    s.v_stride[i] = kst[i];
  }
  s.softmax_scale = 1.0f;
  const int keep = attn_keep_blocks(kNk, kPrefixLen / kBlock, 50);

  // Host inputs.
  const size_t nq_el = (size_t)kQLen * kHq * kD, nk_el = (size_t)kKvLen * kHkv * kD;
  std::vector<uint16_t> hq(nq_el, kNaN), hk(nk_el, kNaN), hv(nk_el, kNaN);
  for (int t = 0; t < kQValid; ++t)
    for (int h = 0; h < kHq; ++h)
      for (int d = 0; d < kD; ++d)
        hq[((size_t)t * kHq + h) * kD + d] = bf16_of(d == target_rank(t, h) ? 16.0f : 0.0f);
  for (int p = 0; p < kKvLen; ++p) {
    const int r = rank_of_pos(p);
    if (r < 0) continue;
    for (int d = 0; d < kD; ++d) {
      hk[(size_t)p * kD + d] = bf16_of(d == r ? 16.0f : 0.0f);
      hv[(size_t)p * kD + d] = bf16_of(value_at(p, d));
    }
  }

  // Device buffers, carved from one allocation at 256-byte offsets.
  const size_t ws_bytes = attn_select_workspace_size(&s);
  if (ws_bytes == 0) return bsattn::report(ATTN_ERR_SELF_TEST, fn, "workspace size query failed");
  auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t n_rows = (size_t)kHq * kNq;
  const size_t off_q = 0, off_k = off_q + r256(nq_el * 2), off_v = off_k + r256(nk_el * 2);
  const size_t off_o = off_v + r256(nk_el * 2), off_lse = off_o + r256(nq_el * 2);
  const size_t off_idx = off_lse + r256((size_t)kHq * kQLen * 4);
  const size_t off_cnt = off_idx + r256(n_rows * kRowStride * 4);
  const size_t off_ws = off_cnt + r256(n_rows * 4), total = off_ws + r256(ws_bytes);
  DeviceBuffers buf;
  char msg[512];
  hipError_t e = hipMalloc(&buf.base, total);
  if (e != hipSuccess) {
    buf.base = nullptr;
    snprintf(msg, sizeof msg, "%s: hipMalloc of %zu bytes failed: %s", where, total,
             hipGetErrorString(e));
    return bsattn::report(ATTN_ERR_DEVICE, fn, msg);
  }
  char* base = static_cast<char*>(buf.base);
  void *dq = base + off_q, *dk = base + off_k, *dv = base + off_v, *dout = base + off_o;
  float* dlse = reinterpret_cast<float*>(base + off_lse);
  int32_t* didx = reinterpret_cast<int32_t*>(base + off_idx);
  int32_t* dcnt = reinterpret_cast<int32_t*>(base + off_cnt);
  if ((e = hipMemcpy(dq, hq.data(), nq_el * 2, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(dk, hk.data(), nk_el * 2, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(dv, hv.data(), nk_el * 2, hipMemcpyHostToDevice)) != hipSuccess) {
    snprintf(msg, sizeof msg, "%s: copy to the device failed: %s", where, hipGetErrorString(e));
    return bsattn::report(ATTN_ERR_DEVICE, fn, msg);
  }

  std::vector<uint16_t> out(nq_el);
  std::vector<float> lse((size_t)kHq * kQLen);
  auto fetch = [&](bool with_lse) -> hipError_t {
    hipError_t r = hipDeviceSynchronize();
    if (r == hipSuccess) r = hipMemcpy(out.data(), dout, nq_el * 2, hipMemcpyDeviceToHost);
    if (r == hipSuccess && with_lse)
      r = hipMemcpy(lse.data(), dlse, lse.size() * 4, hipMemcpyDeviceToHost);
    return r;
  };
  // A failing entry point has set its own message; prefix the device.
  auto propagate = [&](attn_status st, const char* step) {
    snprintf(msg, sizeof msg, "%s: %s returned %d: %s", where, step, (int)st, attn_last_error());
    return bsattn::report(st, fn, msg);
  };
  auto device_error = [&](hipError_t r, const char* step) {
    snprintf(msg, sizeof msg, "%s: %s: %s", where, step, hipGetErrorString(r));
    return bsattn::report(ATTN_ERR_DEVICE, fn, msg);
  };
  auto wrong = [&](const Checker& c) {
    snprintf(msg, sizeof msg, "%s: %s", where, c.msg);
    return bsattn::report(ATTN_ERR_SELF_TEST, fn, msg);
  };

  // 1. Selection: count, order, range, protected block, -1 fill.
  attn_status st = attn_select_blocks(&s, dq, dk, keep, didx, dcnt, kRowStride, base + off_ws,
                                      ws_bytes, nullptr);
  if (st != ATTN_OK) return propagate(st, "attn_select_blocks");
  std::vector<int32_t> idx(n_rows * kRowStride), cnt(n_rows);
  if ((e = hipDeviceSynchronize()) != hipSuccess ||
      (e = hipMemcpy(idx.data(), didx, idx.size() * 4, hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(cnt.data(), dcnt, cnt.size() * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return device_error(e, "selection");
  Checker c;
  for (size_t row = 0; row < n_rows && !c.failed; ++row) {
    const int32_t* li = idx.data() + row * kRowStride;
    if (cnt[row] != keep) {
      snprintf(c.msg, sizeof c.msg, "selection row %zu: count %d, expected %d", row, cnt[row], keep);
      c.failed = true;
      break;
    }
    if (li[0] != 0) c.fail_msg("selection: the protected block is not listed first");
    for (int n = 1; n < keep; ++n)
      if (!(li[n] > li[n - 1] && li[n] < kNk)) c.fail_msg("selection: list not ascending in [0, NK)");
    for (int n = keep; n < kRowStride; ++n)
      if (li[n] != -1) c.fail_msg("selection: unused slot is not -1");
  }
  if (c.failed) return wrong(c);

  // 2. Sparse attention over that list.
  st = attn_block_sparse_fwd(&s, dq, dk, dv, didx, dcnt, kRowStride, dout, nullptr, nullptr);
  if (st != ATTN_OK) return propagate(st, "attn_block_sparse_fwd");
  if ((e = fetch(false)) != hipSuccess) return device_error(e, "sparse attention");
  for (int h = 0; h < kHq; ++h)
    for (int t = 0; t < kQValid; ++t) {
      const int32_t* li = idx.data() + ((size_t)h * kNq + t / kBlock) * kRowStride;
      expect_row(c, "sparse attention", out, h, t, [&](int r) {
        const int j = pos_of_rank(r) / kBlock;
        for (int n = 0; n < keep; ++n)
          if (li[n] == j) return true;
        return false;
      });
    }
  expect_padded_rows_zero(c, "sparse attention, padded row", out);
  if (c.failed) return wrong(c);

  // 3. Dense attention: every row's target is visible; lse = 256.
  st = attn_dense_fwd(&s, dq, dk, dv, dout, dlse, nullptr);
  if (st != ATTN_OK) return propagate(st, "attn_dense_fwd");
  if ((e = fetch(true)) != hipSuccess) return device_error(e, "dense attention");
  for (int h = 0; h < kHq; ++h)
    for (int t = 0; t < kQLen; ++t) {
      if (t < kQValid) expect_row(c, "dense attention", out, h, t, [](int) { return true; });
      const float l = lse[(size_t)h * kQLen + t];
      const bool good = t < kQValid ? std::fabs(l - 256.0f) <= 1e-3f : (std::isinf(l) && l < 0);
      if (!good) c.fail_at("dense attention lse", h, t, -1, l, t < kQValid ? 256.0 : -INFINITY);
    }
  expect_padded_rows_zero(c, "dense attention, padded row", out);
  if (c.failed) return wrong(c);

  // 4. Causal dense attention, aligned at the bottom right over the real
  //    tokens: real row t sees the key ranks up to t + 128 - 100.
  st = attn_dense_causal_fwd(&s, dq, dk, dv, dout, nullptr, nullptr);
  if (st != ATTN_OK) return propagate(st, "attn_dense_causal_fwd");
  if ((e = fetch(false)) != hipSuccess) return device_error(e, "causal attention");
  const int n_real = kPrefixValid + kSuffixValid;
  for (int h = 0; h < kHq; ++h)
    for (int t = 0; t < kQValid; ++t)
      expect_row(c, "causal attention", out, h, t,
                 [&](int r) { return r <= t + n_real - kQValid; });
  expect_padded_rows_zero(c, "causal attention, padded row", out);
  if (c.failed) return wrong(c);

  return bsattn::report(ATTN_OK, fn, "");
}
