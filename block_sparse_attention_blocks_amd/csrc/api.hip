// Host side of libbsattn: argument validation, workspace layout, launches,
// error reporting. The C ABI is declared in include/bsattn.h.
//
// Contract points taken from the pages: the selector lists KV blocks (and
// their number) for every query head and query block and the backend runs
// exactly that list; an error reaches the caller and is never answered with
// dense attention or repeated K/V heads; sparse capability is
// checked on its own (vllm-omni PR #8335 "[Core] Add shared block-sparse
// attention adapters with FlashAttention-4", Purpose). A failure names what
// failed, the library version and the target (in the spirit of the startup
// check of mstar PR #927, "Since the review").

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "bsattn.h"
#include "internal.h"
#include "listcheck.h"

// Builds compiled with BSATTN_CHECK_LISTS=1 (libbsattn_checked.so) validate
// every real query block's list on the device before block-sparse attention.
#ifndef BSATTN_CHECK_LISTS
#define BSATTN_CHECK_LISTS 0
#endif

#define BSATTN_VERSION "0.1.0"
#define BSATTN_TARGET "gfx950"

namespace {

thread_local std::string t_last_error;

attn_status fail(attn_status st, const char* fn, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  char full[768];
  snprintf(full, sizeof full, "%s: %s [libbsattn %s, %s]", fn, msg, BSATTN_VERSION, BSATTN_TARGET);
  t_last_error = full;
  return st;
}

attn_status ok() {
  t_last_error.clear();
  return ATTN_OK;
}

}  // namespace

namespace bsattn {

attn_status report(attn_status st, const char* fn, const char* msg) {
  if (st == ATTN_OK) return ok();
  return fail(st, fn, "%s", msg);
}

}  // namespace bsattn

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Attention workgroups per query block: a workgroup covers at most 128 rows.
int qparts_of(const attn_shape* s) { return s->block_q > 128 ? s->block_q / 128 : 1; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bytes from the first element of a (batch, head) slice of K or V to one
// past its last: kv_len rows `row_stride` elements apart, head_dim each.
int64_t kv_span_bytes(int32_t kv_len, int64_t row_stride, int32_t head_dim) {
  if (kv_len <= 0) return 0;
  return ((int64_t)(kv_len - 1) * row_stride + head_dim) * 2;
}

// Everything about the shape that the kernels rely on.
attn_status validate_shape(const attn_shape* s, const char* fn) {
  if (s == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, "shape is NULL");
  if (s->batch < 1) return fail(ATTN_ERR_INVALID_ARG, fn, "batch %d < 1", s->batch);
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(ATTN_ERR_INVALID_ARG, fn, "head counts must be >= 1 (Hq %d, Hkv %d)",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(ATTN_ERR_INVALID_ARG, fn, "num_q_heads %d is not a multiple of num_kv_heads %d",
                s->num_q_heads, s->num_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "head_dim %d unsupported (supported: 64, 128)",
                s->head_dim);
  if ((s->block_q != 64 && s->block_q != 128 && s->block_q != 256) ||
      (s->block_k != 64 && s->block_k != 128))
    return fail(ATTN_ERR_UNSUPPORTED, fn,
                "block geometry %dx%d unsupported (block_q in {64, 128, 256}, block_k in {64, 128})",
                s->block_q, s->block_k);
  if (s->q_len < 0 || s->q_len % s->block_q != 0)
    return fail(ATTN_ERR_INVALID_ARG, fn, "q_len %d is not a non-negative multiple of block_q %d",
                s->q_len, s->block_q);
  if (s->q_valid < 0 || s->q_valid > s->q_len)
    return fail(ATTN_ERR_INVALID_ARG, fn, "q_valid %d outside [0, q_len %d]", s->q_valid, s->q_len);
  if (s->kv_prefix_len < 0 || s->kv_prefix_len % s->block_k != 0)
    return fail(ATTN_ERR_INVALID_ARG, fn,
                "kv_prefix_len %d is not a non-negative multiple of block_k %d", s->kv_prefix_len,
                s->block_k);
  if (s->kv_prefix_valid < 0 || s->kv_prefix_valid > s->kv_prefix_len)
    return fail(ATTN_ERR_INVALID_ARG, fn, "kv_prefix_valid %d outside [0, kv_prefix_len %d]",
                s->kv_prefix_valid, s->kv_prefix_len);
  if (s->kv_len < s->kv_prefix_len || s->kv_len % s->block_k != 0)
    return fail(ATTN_ERR_INVALID_ARG, fn,
                "kv_len %d must be a multiple of block_k %d and >= kv_prefix_len %d", s->kv_len,
                s->block_k, s->kv_prefix_len);
  if (s->kv_suffix_valid < 0 || s->kv_suffix_valid > s->kv_len - s->kv_prefix_len)
    return fail(ATTN_ERR_INVALID_ARG, fn, "kv_suffix_valid %d outside [0, kv_len - kv_prefix_len = %d]",
                s->kv_suffix_valid, s->kv_len - s->kv_prefix_len);
  const int64_t* strides[4] = {s->q_stride, s->k_stride, s->v_stride, s->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int a = 0; a < 4; ++a)
    for (int d = 0; d < 3; ++d)
      if (strides[a][d] < 0 || strides[a][d] % 8 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, fn,
                    "%s_stride[%d] = %lld must be a non-negative multiple of 8 elements", names[a],
                    d, (long long)strides[a][d]);
  if (!(std::isfinite(s->softmax_scale)))
    return fail(ATTN_ERR_INVALID_ARG, fn, "softmax_scale is not finite");
  if (s->batch > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "batch %d > 65535", s->batch);
  // The attention kernel addresses one (batch, KV head) of K and V with
  // 32-bit byte offsets and packs a block's first key row into 23 bits.
  if (s->kv_len > (1 << 23))
    return fail(ATTN_ERR_UNSUPPORTED, fn, "kv_len %d > %d", s->kv_len, 1 << 23);
  // The attention kernel addresses one KV head's rows through a buffer
  // resource of 31-bit range that starts up to 3 KB before them.
  if (kv_span_bytes(s->kv_len, s->k_stride[1], s->head_dim) > 0x7FFFFFFF - 4096 ||
      kv_span_bytes(s->kv_len, s->v_stride[1], s->head_dim) > 0x7FFFFFFF - 4096)
    return fail(ATTN_ERR_UNSUPPORTED, fn,
                "one KV head spans more than 2 GiB (kv_len %d, k row stride %lld, v row stride %lld)",
                s->kv_len, (long long)s->k_stride[1], (long long)s->v_stride[1]);
  const int64_t nwg = (int64_t)s->batch * s->num_q_heads * (s->q_len / s->block_q) * qparts_of(s);
  // (+ up to 7 padding workgroups per (batch, KV head) in the head-synchronous order)
  if (nwg + 8 * (int64_t)s->batch * s->num_kv_heads > 0x7FFFFFFF)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "grid too large");
  return ATTN_OK;
}

attn_status validate_ptr(const char* fn, const char* name, const void* ptr) {
  if (ptr == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(ATTN_ERR_UNSUPPORTED, fn, "%s is not 16-byte aligned", name);
  return ATTN_OK;
}

attn_status validate_tensors(const char* fn, const void* q, const void* k, const void* v,
                             const void* o, const float* lse) {
  attn_status st;
  if ((st = validate_ptr(fn, "q", q)) != ATTN_OK) return st;
  if ((st = validate_ptr(fn, "k", k)) != ATTN_OK) return st;
  if ((st = validate_ptr(fn, "v", v)) != ATTN_OK) return st;
  if ((st = validate_ptr(fn, "out", o)) != ATTN_OK) return st;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(ATTN_ERR_INVALID_ARG, fn, "lse is not 4-byte aligned");
  return ATTN_OK;
}

// The current device must be a gfx950; the answer is cached per device.
attn_status check_device(const char* fn) {
  static std::atomic<int> state[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(ATTN_ERR_DEVICE, fn, "no HIP device available");
  if (dev >= 64) return fail(ATTN_ERR_DEVICE, fn, "device ordinal %d too large", dev);
  int st = state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(ATTN_ERR_DEVICE, fn, "cannot query device %d", dev);
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    state[dev].store(st, std::memory_order_relaxed);
    if (st < 0)
      return fail(ATTN_ERR_DEVICE, fn, "device %d is %s, this library runs on gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (st < 0) return fail(ATTN_ERR_DEVICE, fn, "device %d is not a gfx950", dev);
  return ATTN_OK;
}

struct Derived {
  int nq, nk, P, n_forced, n_cand, group;
};

Derived derive(const attn_shape* s) {
  Derived d;
  d.nq = s->q_len / s->block_q;
  d.nk = s->kv_len / s->block_k;
  d.P = s->kv_prefix_len / s->block_k;
  d.n_forced = (int)ceil_div(s->kv_prefix_valid, s->block_k);
  d.n_cand = (int)ceil_div(s->kv_suffix_valid, s->block_k);
  d.group = s->num_q_heads / s->num_kv_heads;
  return d;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qp, qn, kpt, kn, total;
};

WsLayout ws_layout(const attn_shape* s) {
  const Derived d = derive(s);
  const size_t B = (size_t)s->batch, D = (size_t)s->head_dim;
  WsLayout w;
  w.qp = 0;
  w.qn = w.qp + round256(B * s->num_q_heads * d.nq * D * sizeof(double));
  w.kpt = w.qn + round256(B * s->num_q_heads * d.nq * sizeof(double));
  w.kn = w.kpt + round256(B * s->num_kv_heads * D * d.nk * sizeof(float));
  w.total = w.kn + round256(B * s->num_kv_heads * d.nk * sizeof(double));
  return w;
}

float scale_of(const attn_shape* s) {
  return s->softmax_scale > 0.0f ? s->softmax_scale : 1.0f / std::sqrt((float)s->head_dim);
}

#if BSATTN_CHECK_LISTS
// The first faulty list, as ((row << 32) | ((slot + 1) << 2) | fault): the
// smallest row wins, so the report does not depend on the schedule.
__device__ unsigned long long g_list_fault;

constexpr int kCheckRows = 64;         // rows per workgroup, one per thread
constexpr int kCheckMaxBlocks = 4096;  // KV blocks a thread's LDS bitmap covers

__global__ void __launch_bounds__(kCheckRows)
check_lists_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                   int32_t stride, int32_t nk, int32_t nq, int32_t real_qblocks, int64_t rows) {
  __shared__ uint32_t seen[kCheckRows][kCheckMaxBlocks / 32];
  const int64_t row = (int64_t)blockIdx.x * kCheckRows + threadIdx.x;
  if (row >= rows || (int32_t)(row % nq) >= real_qblocks) return;
  int32_t pos = -1;
  const int32_t f =
      bsattn::check_list_row(idx + row * stride, cnt[row], stride, nk,
                             nk <= kCheckMaxBlocks ? seen[threadIdx.x] : nullptr, &pos);
  if (f != bsattn::kListOk) {
    const unsigned long long key = ((unsigned long long)row << 32) |
                                   ((unsigned long long)(uint32_t)(pos + 1) << 2) |
                                   (unsigned long long)f;
    atomicMin(&g_list_fault, key);
  }
}

// Runs the list check on `stream` and waits for it. Rows of query blocks with
// no real query row are not read by the attention kernel and not checked.
attn_status check_lists(const char* fn, const attn_shape* s, const Derived& d, const int32_t* idx,
                        const int32_t* cnt, int32_t stride, hipStream_t stream) {
  const int64_t rows = (int64_t)s->batch * s->num_q_heads * d.nq;
  const int32_t real_qblocks = (int32_t)ceil_div(s->q_valid, s->block_q);
  const unsigned long long none = ~0ull;
  unsigned long long got = none;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_list_fault), &none, sizeof none, 0,
                                        hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) {
    const int64_t grid = (rows + kCheckRows - 1) / kCheckRows;
    hipLaunchKernelGGL(check_lists_kernel, dim3((unsigned)grid), dim3(kCheckRows), 0, stream, idx,
                       cnt, stride, d.nk, d.nq, real_qblocks, rows);
    e = hipGetLastError();
  }
  if (e == hipSuccess)
    e = hipMemcpyFromSymbolAsync(&got, HIP_SYMBOL(g_list_fault), sizeof got, 0,
                                 hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, fn, "list check failed: %s", hipGetErrorString(e));
  if (got == none) return ATTN_OK;
  const int64_t row = (int64_t)(got >> 32);
  const int32_t slot = (int32_t)((got >> 2) & 0x3FFFFFFFu) - 1;
  const int32_t fault = (int32_t)(got & 3u);
  const int32_t i = (int32_t)(row % d.nq);
  const int32_t h = (int32_t)((row / d.nq) % s->num_q_heads);
  const int32_t b = (int32_t)(row / d.nq / s->num_q_heads);
  int32_t count = 0, entry = 0;
  (void)hipMemcpy(&count, cnt + row, sizeof count, hipMemcpyDeviceToHost);
  if (slot >= 0) (void)hipMemcpy(&entry, idx + row * stride + slot, sizeof entry, hipMemcpyDeviceToHost);
  if (fault == bsattn::kListCount)
    return fail(ATTN_ERR_INVALID_ARG, fn,
                "block list of (batch %d, head %d, query block %d): count %d outside [0, %d]", b, h,
                i, count, stride);
  if (fault == bsattn::kListRange)
    return fail(ATTN_ERR_INVALID_ARG, fn,
                "block list of (batch %d, head %d, query block %d): entry %d is %d, outside [0, %d)",
                b, h, i, slot, entry, d.nk);
  return fail(ATTN_ERR_INVALID_ARG, fn,
              "block list of (batch %d, head %d, query block %d): entry %d repeats block %d", b, h,
              i, slot, entry);
}
#endif

attn_status run_attention(const char* fn, const attn_shape* s, const void* q, const void* k,
                          const void* v, const int32_t* idx, const int32_t* cnt,
                          int32_t idx_row_stride, void* out, float* lse, int mode,
                          hipStream_t stream) {
  const bool dense = mode != bsattn::kSparse;
  attn_status st = validate_shape(s, fn);
  if (st != ATTN_OK) return st;
  st = validate_tensors(fn, q, k, v, out, lse);
  if (st != ATTN_OK) return st;
  if (!dense) {
    if (idx == nullptr || cnt == nullptr)
      return fail(ATTN_ERR_INVALID_ARG, fn, "block_idx / block_cnt is NULL");
    if ((reinterpret_cast<uintptr_t>(idx) & 3u) || (reinterpret_cast<uintptr_t>(cnt) & 3u))
      return fail(ATTN_ERR_INVALID_ARG, fn, "block_idx / block_cnt not 4-byte aligned");
    if (idx_row_stride < 1)
      return fail(ATTN_ERR_INVALID_ARG, fn, "idx_row_stride %d < 1", idx_row_stride);
  }
  const Derived d = derive(s);
  bsattn::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.idx = idx;
  p.cnt = cnt;
  p.qs0 = s->q_stride[0]; p.qs1 = s->q_stride[1]; p.qs2 = s->q_stride[2];
  p.ks0 = s->k_stride[0]; p.ks1 = s->k_stride[1]; p.ks2 = s->k_stride[2];
  p.vs0 = s->v_stride[0]; p.vs1 = s->v_stride[1]; p.vs2 = s->v_stride[2];
  p.os0 = s->o_stride[0]; p.os1 = s->o_stride[1]; p.os2 = s->o_stride[2];
  p.batch = s->batch;
  p.hq = s->num_q_heads;
  p.hkv = s->num_kv_heads;
  p.group = d.group;
  p.q_len = s->q_len;
  p.q_valid = s->q_valid;
  p.kv_prefix_len = s->kv_prefix_len;
  p.kv_prefix_valid = s->kv_prefix_valid;
  p.kv_suffix_valid = s->kv_suffix_valid;
  p.nq = d.nq;
  p.nk = d.nk;
  p.n_prefix_blocks = d.P;
  p.n_forced = d.n_forced;
  p.n_cand = d.n_cand;
  p.idx_row_stride = dense ? 0 : idx_row_stride;
  p.causal_off = (s->kv_prefix_valid + s->kv_suffix_valid) - s->q_valid;
  p.qparts = qparts_of(s);
  p.n_wg = (int)((int64_t)s->batch * s->num_q_heads * d.nq * p.qparts);
  // K and V of every (batch, KV head) together larger than the 256 MB
  // last-level cache: let the XCDs work through the KV heads in step.
  const int64_t kv_bytes =
      (int64_t)s->batch * s->num_kv_heads * (int64_t)s->kv_len * s->head_dim * 2 * 2;
  p.head_sync = kv_bytes > ((int64_t)256 << 20) ? 1 : 0;
  p.scale_log2 = scale_of(s) * 1.4426950408889634f;
  p.k_span_bytes = (uint32_t)kv_span_bytes(s->kv_len, s->k_stride[1], s->head_dim);
  p.v_span_bytes = (uint32_t)kv_span_bytes(s->kv_len, s->v_stride[1], s->head_dim);
  if (p.n_wg == 0) return ok();
  st = check_device(fn);
  if (st != ATTN_OK) return st;
#if BSATTN_CHECK_LISTS
  if (!dense) {
    st = check_lists(fn, s, d, idx, cnt, idx_row_stride, stream);
    if (st != ATTN_OK) return st;
  }
#endif
  const hipError_t e = bsattn::launch_attention(p, s->head_dim, s->block_q, s->block_k, mode, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, fn, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t attn_keep_blocks(int32_t n_kv_blocks, int32_t n_protected, int32_t sparsity_pct) {
  if (n_kv_blocks < 0 || n_protected < 0 || n_protected > n_kv_blocks || sparsity_pct < 0 ||
      sparsity_pct > 100)
    return -1;
  const int64_t k = ceil_div((int64_t)n_kv_blocks * (100 - sparsity_pct), 100);
  int64_t r = k < n_protected ? n_protected : k;
  if (r > n_kv_blocks) r = n_kv_blocks;
  return (int32_t)r;
}

size_t attn_select_workspace_size(const attn_shape* shape) {
  if (validate_shape(shape, "attn_select_workspace_size") != ATTN_OK) return 0;
  return ws_layout(shape).total;
}

}  // extern "C"

namespace {

attn_status select_impl(const char* fn, const attn_shape* s, const void* q, const void* k,
                        int32_t keep_blocks, int32_t* block_idx, int32_t* block_cnt,
                        int32_t idx_row_stride, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  attn_status st = validate_shape(s, fn);
  if (st != ATTN_OK) return st;
  if ((st = validate_ptr(fn, "q", q)) != ATTN_OK) return st;
  if ((st = validate_ptr(fn, "k", k)) != ATTN_OK) return st;
  const Derived d = derive(s);
  if (keep_blocks < d.P || keep_blocks > d.nk)
    return fail(ATTN_ERR_INVALID_ARG, fn, "keep_blocks %d outside [P = %d, NK = %d]", keep_blocks,
                d.P, d.nk);
  if (idx_row_stride < keep_blocks || idx_row_stride < 1)
    return fail(ATTN_ERR_INVALID_ARG, fn, "idx_row_stride %d < max(keep_blocks %d, 1)",
                idx_row_stride, keep_blocks);
  if (block_idx == nullptr || block_cnt == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, fn, "block_idx / block_cnt is NULL");
  if ((reinterpret_cast<uintptr_t>(block_idx) & 3u) || (reinterpret_cast<uintptr_t>(block_cnt) & 3u))
    return fail(ATTN_ERR_INVALID_ARG, fn, "block_idx / block_cnt not 4-byte aligned");
  if (d.nk > 4096)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "%d KV blocks > 4096 supported by the selector", d.nk);
  const WsLayout w = ws_layout(s);
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(ATTN_ERR_WORKSPACE, fn, "workspace %zu bytes < %zu required", workspace_bytes,
                w.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(ATTN_ERR_WORKSPACE, fn, "workspace is not 256-byte aligned");
  if (d.nq == 0) return ok();
  st = check_device(fn);
  if (st != ATTN_OK) return st;
  char* ws = static_cast<char*>(workspace);

  bsattn::PoolParams pp{};
  pp.q = static_cast<const uint16_t*>(q);
  pp.k = static_cast<const uint16_t*>(k);
  pp.qs0 = s->q_stride[0]; pp.qs1 = s->q_stride[1]; pp.qs2 = s->q_stride[2];
  pp.ks0 = s->k_stride[0]; pp.ks1 = s->k_stride[1]; pp.ks2 = s->k_stride[2];
  pp.hq = s->num_q_heads;
  pp.hkv = s->num_kv_heads;
  pp.bq = s->block_q;
  pp.bk = s->block_k;
  pp.q_valid = s->q_valid;
  pp.kv_prefix_len = s->kv_prefix_len;
  pp.kv_prefix_valid = s->kv_prefix_valid;
  pp.kv_suffix_valid = s->kv_suffix_valid;
  pp.nq = d.nq;
  pp.nk = d.nk;
  pp.qp = reinterpret_cast<double*>(ws + w.qp);
  pp.qn = reinterpret_cast<double*>(ws + w.qn);
  pp.kpt = reinterpret_cast<float*>(ws + w.kpt);
  pp.kn = reinterpret_cast<double*>(ws + w.kn);
  hipError_t e = bsattn::launch_pool(pp, s->head_dim, s->batch, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, fn, "pool launch failed: %s", hipGetErrorString(e));

  bsattn::ScoreParams sp{};
  sp.qp = pp.qp;
  sp.qn = pp.qn;
  sp.kpt = pp.kpt;
  sp.kn = pp.kn;
  sp.idx = block_idx;
  sp.cnt = block_cnt;
  sp.hq = s->num_q_heads;
  sp.hkv = s->num_kv_heads;
  sp.group = d.group;
  sp.nq = d.nq;
  sp.nk = d.nk;
  sp.bq = s->block_q;
  sp.q_valid = s->q_valid;
  sp.n_prefix_blocks = d.P;
  sp.n_forced = d.n_forced;
  sp.n_cand = d.n_cand;
  sp.keep = keep_blocks;
  sp.idx_row_stride = idx_row_stride;
  e = bsattn::launch_score_topk(sp, s->head_dim, s->batch, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, fn, "score launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Scratch of attn_select_blocks_noalloc: one array per device that holds the
// pooled vectors, for callers that cannot allocate. Host code never uses the
// array's name as an address: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept here.
constexpr size_t kStaticWorkspaceBytes = (size_t)ATTN_SELECT_STATIC_WORKSPACE_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticWorkspaceBytes];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[64] = {};

attn_status static_workspace(const char* fn, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(ATTN_ERR_DEVICE, fn, "no HIP device available");
  if (dev >= 64) return fail(ATTN_ERR_DEVICE, fn, "device ordinal %d too large", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(ATTN_ERR_DEVICE, fn, "cannot find the scratch array on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_select_blocks(const attn_shape* s, const void* q, const void* k,
                               int32_t keep_blocks, int32_t* block_idx, int32_t* block_cnt,
                               int32_t idx_row_stride, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return select_impl("attn_select_blocks", s, q, k, keep_blocks, block_idx, block_cnt,
                     idx_row_stride, workspace, workspace_bytes, stream);
}

attn_status attn_select_blocks_noalloc(const attn_shape* s, const void* q, const void* k,
                                       int32_t keep_blocks, int32_t* block_idx,
                                       int32_t* block_cnt, int32_t idx_row_stride,
                                       hipStream_t stream) {
  const char* fn = "attn_select_blocks_noalloc";
  attn_status st = validate_shape(s, fn);
  if (st != ATTN_OK) return st;
  const size_t need = ws_layout(s).total;
  if (need > kStaticWorkspaceBytes)
    return fail(ATTN_ERR_WORKSPACE, fn,
                "the shape needs %zu bytes of selector workspace, the library's fixed array holds "
                "%zu (use attn_select_blocks with a caller workspace)",
                need, kStaticWorkspaceBytes);
  if ((st = check_device(fn)) != ATTN_OK) return st;
  void* ws = nullptr;
  if ((st = static_workspace(fn, &ws)) != ATTN_OK) return st;
  return select_impl(fn, s, q, k, keep_blocks, block_idx, block_cnt, idx_row_stride, ws,
                     kStaticWorkspaceBytes, stream);
}

attn_status attn_block_sparse_fwd(const attn_shape* s, const void* q, const void* k, const void* v,
                                  const int32_t* block_idx, const int32_t* block_cnt,
                                  int32_t idx_row_stride, void* out, float* lse,
                                  hipStream_t stream) {
  return run_attention("attn_block_sparse_fwd", s, q, k, v, block_idx, block_cnt, idx_row_stride,
                       out, lse, bsattn::kSparse, stream);
}

attn_status attn_dense_fwd(const attn_shape* s, const void* q, const void* k, const void* v,
                           void* out, float* lse, hipStream_t stream) {
  return run_attention("attn_dense_fwd", s, q, k, v, nullptr, nullptr, 0, out, lse, bsattn::kDense,
                       stream);
}

attn_status attn_dense_causal_fwd(const attn_shape* s, const void* q, const void* k, const void* v,
                                  void* out, float* lse, hipStream_t stream) {
  return run_attention("attn_dense_causal_fwd", s, q, k, v, nullptr, nullptr, 0, out, lse,
                       bsattn::kCausal, stream);
}

attn_status attn_query_support(const attn_shape* s) {
  const char* fn = "attn_query_support";
  const attn_status st = validate_shape(s, fn);
  if (st != ATTN_OK) return st;
  if (derive(s).nk > 4096)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "%d KV blocks > 4096 supported by the selector",
                derive(s).nk);
  return ok();
}

// ------------------------------------------------------------- strategy
int32_t attn_strategy_is_sparse(const attn_strategy* st, int32_t step, int32_t layer) {
  if (st == nullptr || st->num_layers < 1 || st->num_layers > 64 || st->dense_steps < 0 ||
      st->sparsity_pct < 0 || st->sparsity_pct > 100 || step < 0 || layer < 0 ||
      layer >= st->num_layers)
    return -1;
  if (st->num_layers < 64 && (st->sparse_layers >> st->num_layers) != 0) return -1;
  if (step < st->dense_steps) return 0;
  return (int32_t)((st->sparse_layers >> layer) & 1u);
}

}  // extern "C"

namespace {

// Workspace of a strategy call: block lists, counts, then the selector's.
struct StrategyWs {
  int32_t keep;
  size_t idx, cnt, sel, total;
};

bool strategy_ws(const attn_shape* s, const attn_strategy* st, StrategyWs* w) {
  if (validate_shape(s, "attn_strategy") != ATTN_OK) return false;
  if (attn_strategy_is_sparse(st, 0, 0) < 0) return false;
  const Derived d = derive(s);
  w->keep = attn_keep_blocks(d.nk, d.P, st->sparsity_pct);
  if (w->keep < 0) return false;
  const size_t rows = (size_t)s->batch * s->num_q_heads * d.nq;
  w->idx = 0;
  w->cnt = round256(rows * (size_t)(w->keep > 0 ? w->keep : 1) * sizeof(int32_t));
  w->sel = w->cnt + round256(rows * sizeof(int32_t));
  w->total = w->sel + ws_layout(s).total;
  return true;
}

attn_status strategy_call(const char* fn, const attn_shape* s, const attn_strategy* st,
                          bool sparse, const void* q, const void* k, const void* v, void* out,
                          float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!sparse) return attn_dense_fwd(s, q, k, v, out, lse, stream);
  StrategyWs w;
  if (!strategy_ws(s, st, &w)) return fail(ATTN_ERR_INVALID_ARG, fn, "invalid shape or strategy");
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(ATTN_ERR_WORKSPACE, fn, "workspace %zu bytes < %zu required", workspace_bytes,
                w.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(ATTN_ERR_WORKSPACE, fn, "workspace is not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + w.idx);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
  const int32_t stride = w.keep > 0 ? w.keep : 1;
  attn_status r = attn_select_blocks(s, q, k, w.keep, idx, cnt, stride, ws + w.sel,
                                     workspace_bytes - w.sel, stream);
  if (r != ATTN_OK) return r;
  return attn_block_sparse_fwd(s, q, k, v, idx, cnt, stride, out, lse, stream);
}

}  // namespace

extern "C" {

size_t attn_strategy_workspace_size(const attn_shape* s, const attn_strategy* st) {
  StrategyWs w;
  return strategy_ws(s, st, &w) ? w.total : 0;
}

attn_status attn_strategy_fwd(const attn_shape* s, const attn_strategy* st, int32_t step,
                              int32_t layer, const void* q, const void* k, const void* v,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  const char* fn = "attn_strategy_fwd";
  const int32_t sp = attn_strategy_is_sparse(st, step, layer);
  if (sp < 0)
    return fail(ATTN_ERR_INVALID_ARG, fn, "invalid strategy or (step %d, layer %d)", step, layer);
  return strategy_call(fn, s, st, sp == 1, q, k, v, out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_strategy_warmup(const attn_shape* s, const attn_strategy* st, const void* q,
                                 const void* k, const void* v, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "attn_strategy_warmup";
  if (attn_strategy_is_sparse(st, 0, 0) < 0) return fail(ATTN_ERR_INVALID_ARG, fn, "invalid strategy");
  const uint64_t all = st->num_layers == 64 ? ~0ull : ((1ull << st->num_layers) - 1);
  const bool any_dense = st->dense_steps > 0 || (st->sparse_layers & all) != all;
  const bool any_sparse = st->sparse_layers != 0;
  if (any_dense) {
    const attn_status r =
        strategy_call(fn, s, st, false, q, k, v, out, nullptr, workspace, workspace_bytes, stream);
    if (r != ATTN_OK) return r;
  }
  if (any_sparse) {
    const attn_status r =
        strategy_call(fn, s, st, true, q, k, v, out, nullptr, workspace, workspace_bytes, stream);
    if (r != ATTN_OK) return r;
  }
  return ok();
}

const char* attn_last_error(void) { return t_last_error.c_str(); }

const char* attn_version(void) { return BSATTN_VERSION; }

}  // extern "C"
